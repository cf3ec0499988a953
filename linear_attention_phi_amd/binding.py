"""Thin ctypes binding of ``include/linattn.h`` for torch tensors.

Argument marshalling only: shapes and dtypes are checked, device pointers and
the current HIP stream are handed to the C ABI, and every step of the method
runs in the HIP library.  There is no fallback: if ``liblinattn.so`` is
missing, or a call returns an error status, a RuntimeError is raised.

The C ABI receives bare pointers and cannot see a tensor's size, so every
tensor a caller passes (inputs, initial states and preallocated outputs alike)
is checked here against the shape the call implies, before anything is
launched: first the shapes and dtypes of all of them (ValueError / TypeError),
then that each is a contiguous tensor on the GPU.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
PHI_ELU1, PHI_IDENTITY = 0, 1
KIND_FORWARD, KIND_GATED, KIND_NONCAUSAL, KIND_BACKWARD, KIND_TRAIN = 0, 1, 2, 3, 4

_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (argtypes, restype), in the order of include/linattn.h
SIGNATURES = {
    "linattn_forward": ([_P] * 8 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_forward_gated": ([_P] * 9 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_forward_noalloc": ([_P] * 8 + [_I] * 7 + [_F, _P], _I),
    "linattn_forward_planned": ([_P] * 9 + [_I] * 7 + [_F, _I, _I, _P, _SZ, _P], _I),
    "linattn_forward_train": ([_P] * 9 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_backward": ([_P] * 11 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_decode_step_lowp": ([_P] * 5 + [_I] + [_P] * 2 + [_I] * 6 + [_F, _P], _I),
    "linattn_forward_delta": ([_P] * 8 + [_I] * 7 + [_P], _I),
    "linattn_forward_snapshots": ([_P] * 10 + [_I] + [_P] * 2 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_forward_noncausal": ([_P] * 6 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_decode_step": ([_P] * 7 + [_I] * 6 + [_F, _P], _I),
    "linattn_workspace_size": ([_I] * 7, _SZ),
    "linattn_workspace_size_planned": ([_I] * 9, _SZ),
    "linattn_status_string": ([_I], ctypes.c_char_p),
    "linattn_abi_version": ([], _I),
    "linattn_profile_enable": ([_I], _I),
    "linattn_profile_read": ([_P, _P, _P, _I], _I),
}


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m linear_attention_phi_amd.build` "
                    "(there is no non-HIP fallback)")
            h = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.argtypes = args
                fn.restype = res
            _lib = h
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().linattn_status_string(rc).decode()
        raise RuntimeError(f"{what} failed: {msg} ({rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dims(t, name, ndim):
    """The shape of the tensor that fixes a call's sizes (q), checked for rank only."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _validate(specs):
    """specs: (tensor or None, name, expected shape, expected dtype or None).

    Shapes and dtypes of every given tensor first, then device and layout, so
    that a wrong size is reported whatever device the tensors are on and
    nothing reaches the GPU before all of it has passed.
    """
    for t, name, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    for t, name, _, _ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _pair(a, b, what):
    if (a is None) != (b is None):
        raise ValueError(f"pass both {what} or neither")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def workspace_size(kind, B, H, N, Dk, Dv, dtype_code) -> int:
    return int(lib().linattn_workspace_size(kind, B, H, N, Dk, Dv, dtype_code))


def workspace_size_planned(kind, B, H, N, Dk, Dv, dtype_code, segments, subsegments) -> int:
    return int(lib().linattn_workspace_size_planned(kind, B, H, N, Dk, Dv, dtype_code, segments, subsegments))


def _workspace(need, device, workspace):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _validate([(workspace, "workspace", tuple(workspace.shape), None)])
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {need}")
    return workspace


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


def _qkv_specs(q, k, v):
    """Sizes fixed by q and v, and the specs of q, k, v themselves."""
    B, H, N, Dk = _dims(q, "q", 4)
    Dv = _dims(v, "v", 4)[3]
    code = _dtype_code(q)
    return (B, H, N, Dk, Dv, code), [(q, "q", (B, H, N, Dk), None), (k, "k", (B, H, N, Dk), q.dtype),
                                     (v, "v", (B, H, N, Dv), q.dtype)]


def linattn_forward(q, k, v, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, want_state=True,
                    out=None, s_final=None, z_final=None, workspace=None):
    """Causal forward.  q, k [B, H, N, Dk]; v [B, H, N, Dv] -> (o, s_final, z_final)."""
    return _forward(None, q, k, v, None, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace)


def linattn_forward_gated(q, k, v, alpha, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1,
                          want_state=True, out=None, s_final=None, z_final=None, workspace=None):
    """Gated causal forward with alpha [B, H, N] fp32 -> (o, s_final, z_final)."""
    if alpha is None:
        raise ValueError("alpha is required")
    return _forward(None, q, k, v, alpha, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace)


def linattn_forward_planned(q, k, v, segments, subsegments, alpha=None, s_init=None, z_init=None, *, eps=1e-6,
                            phi=PHI_ELU1, want_state=True, out=None, s_final=None, z_final=None, workspace=None):
    """Causal forward (gated if alpha is given) with the sequence split into at most `segments` output
    segments of `subsegments` state parts each -> (o, s_final, z_final)."""
    return _forward((int(segments), int(subsegments)), q, k, v, alpha, s_init, z_init, eps, phi, want_state, out,
                    s_final, z_final, workspace)


NOALLOC_SCRATCH_BYTES = 48 << 20


def linattn_forward_noalloc(q, k, v, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, out=None,
                            s_final=None, z_final=None):
    """linattn_forward without a workspace: the library's fixed device scratch holds the segment states.

    The C call allocates nothing; pass ``out`` (and ``s_final``, ``z_final``
    to receive the state) to allocate nothing here either.  Calls that overlap
    in time on one GPU share the scratch and race.  Raises if the sizes need
    more than NOALLOC_SCRATCH_BYTES of segment states.
    """
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _pair(s_init, z_init, "s_init and z_init")
    _pair(s_final, z_final, "s_final and z_final")
    need = workspace_size(KIND_FORWARD, B, H, N, Dk, Dv, code)
    if need > NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"these sizes need {need} bytes of segment states; the fixed scratch holds "
                         f"{NOALLOC_SCRATCH_BYTES} (use linattn_forward with a workspace)")
    _validate(specs + [(s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (z_init, "z_init", (B, H, Dk), torch.float32),
                       (out, "out", (B, H, N, Dv), q.dtype),
                       (s_final, "s_final", (B, H, Dk, Dv), torch.float32),
                       (z_final, "z_final", (B, H, Dk), torch.float32)])
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    rc = lib().linattn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s_init), _ptr(z_init),
                                       _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps),
                                       _stream(q))
    _check(rc, "linattn_forward_noalloc")
    return o, s_final, z_final


def _forward(plan, q, k, v, alpha, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace):
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _pair(s_init, z_init, "s_init and z_init")
    _pair(s_final, z_final, "s_final and z_final")
    _validate(specs + [(alpha, "alpha", (B, H, N), torch.float32),
                       (s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (z_init, "z_init", (B, H, Dk), torch.float32),
                       (out, "out", (B, H, N, Dv), q.dtype),
                       (s_final, "s_final", (B, H, Dk, Dv), torch.float32),
                       (z_final, "z_final", (B, H, Dk), torch.float32)])
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    if want_state:
        if s_final is None:
            s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
            z_final = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    else:
        s_final = z_final = None
    gated = alpha is not None
    kind = KIND_GATED if gated else KIND_FORWARD
    L = lib()
    if plan is not None:
        need = workspace_size_planned(kind, B, H, N, Dk, Dv, code, *plan)
        ws = _workspace(need, q.device, workspace)
        rc = L.linattn_forward_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(s_init), _ptr(z_init),
                                       _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps),
                                       plan[0], plan[1], _ptr(ws), _ws_bytes(ws), _stream(q))
        _check(rc, "linattn_forward_planned")
        return o, s_final, z_final
    ws = _workspace(workspace_size(kind, B, H, N, Dk, Dv, code), q.device, workspace)
    if gated:
        rc = L.linattn_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(s_init), _ptr(z_init),
                                     _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps),
                                     _ptr(ws), _ws_bytes(ws), _stream(q))
    else:
        rc = L.linattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s_init), _ptr(z_init), _ptr(s_final),
                               _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws), _ws_bytes(ws),
                               _stream(q))
    _check(rc, "linattn_forward_gated" if gated else "linattn_forward")
    return o, s_final, z_final


def linattn_forward_train(q, k, v, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, workspace=None):
    """Causal forward that also keeps each token's denominator -> (o, den, s_final, z_final, saved).

    bf16 with Dk, Dv in {64, 128}; den [B, H, N] fp32 feeds linattn_backward,
    and so may ``saved`` (the workspace, which then holds the forward state at
    every segment start; pass it to linattn_backward unchanged).
    """
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _pair(s_init, z_init, "s_init and z_init")
    _validate(specs + [(s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (z_init, "z_init", (B, H, Dk), torch.float32)])
    o = torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    z_final = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    ws = _workspace(workspace_size(KIND_TRAIN, B, H, N, Dk, Dv, code), q.device, workspace)
    rc = lib().linattn_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _ptr(s_init), _ptr(z_init),
                                     _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws),
                                     _ws_bytes(ws), _stream(q))
    _check(rc, "linattn_forward_train")
    return o, den, s_final, z_final, ws


def linattn_backward(q, k, v, den, dout, s_init=None, z_init=None, *, saved=None, eps=1e-6, phi=PHI_ELU1,
                     out=None, workspace=None):
    """Gradients of a loss through the causal forward, given dout = dL/dO -> (dq, dk, dv).

    den is the output of linattn_forward_train on the same q, k, v (and
    initial state, eps, phi); ``saved``, its workspace (optional: without it
    the segment states are recomputed).  ``out`` may pass preallocated (dq, dk, dv).
    """
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _pair(s_init, z_init, "s_init and z_init")
    if out is not None and len(out) != 3:
        raise ValueError("out must be (dq, dk, dv)")
    dq, dk, dv = out if out is not None else (None, None, None)
    _validate(specs + [(den, "den", (B, H, N), torch.float32), (dout, "dout", (B, H, N, Dv), q.dtype),
                       (s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (z_init, "z_init", (B, H, Dk), torch.float32),
                       (dq, "dq", (B, H, N, Dk), q.dtype), (dk, "dk", (B, H, N, Dk), q.dtype),
                       (dv, "dv", (B, H, N, Dv), q.dtype)])
    if den is None or dout is None:
        raise ValueError("den and dout are required")
    if saved is not None:
        need = workspace_size(KIND_TRAIN, B, H, N, Dk, Dv, code)
        if not isinstance(saved, torch.Tensor) or saved.numel() * saved.element_size() < need:
            raise ValueError(f"saved must be the training forward's workspace ({need} bytes)")
        _validate([(saved, "saved", tuple(saved.shape), None)])
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = _workspace(workspace_size(KIND_BACKWARD, B, H, N, Dk, Dv, code), q.device, workspace)
    rc = lib().linattn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(den), _ptr(saved), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv),
                                _ptr(s_init), _ptr(z_init), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws),
                                _ws_bytes(ws), _stream(q))
    _check(rc, "linattn_backward")
    return dq, dk, dv


def linattn_forward_delta(q, k, v, beta=None, s_init=None, *, alpha=None, phi=PHI_ELU1, want_state=True,
                          out=None):
    """Delta rule: decay the summary by alpha (gated form), read it with the unit key
    phi(k)/|phi(k)|, write beta times the difference, o = S^T phi(q).  alpha, beta [B, H, N]
    fp32 or None (ones) -> (o, s_final or None).  bf16 with Dk, Dv in {64, 128}.
    """
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _validate(specs + [(beta, "beta", (B, H, N), torch.float32), (alpha, "alpha", (B, H, N), torch.float32),
                       (s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (out, "out", (B, H, N, Dv), q.dtype)])
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_state else None
    rc = lib().linattn_forward_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _ptr(s_init),
                                     _ptr(s_final), B, H, N, Dk, Dv, code, phi, _stream(q))
    _check(rc, "linattn_forward_delta")
    return o, s_final


MAX_SNAPSHOTS = 256


def linattn_forward_snapshots(q, k, v, positions, alpha=None, s_init=None, z_init=None, *, eps=1e-6,
                              phi=PHI_ELU1, workspace=None):
    """Causal forward that also returns the state after each listed token.

    positions: ints in [0, N) (at most MAX_SNAPSHOTS) -> (o, s_snap [B, H, n, Dk, Dv],
    z_snap [B, H, n, Dk], s_final, z_final).  alpha [B, H, N] fp32 or None.
    bf16 with Dk, Dv in {64, 128}.
    """
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _pair(s_init, z_init, "s_init and z_init")
    pos = [int(p) for p in positions]
    n = len(pos)
    if not 1 <= n <= MAX_SNAPSHOTS:
        raise ValueError(f"1 to {MAX_SNAPSHOTS} positions")
    if not all(0 <= p < N for p in pos):
        raise ValueError(f"positions must lie in [0, {N})")
    _validate(specs + [(alpha, "alpha", (B, H, N), torch.float32),
                       (s_init, "s_init", (B, H, Dk, Dv), torch.float32),
                       (z_init, "z_init", (B, H, Dk), torch.float32)])
    parr = (ctypes.c_int * n)(*pos)
    o = torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    s_snap = torch.empty((B, H, n, Dk, Dv), dtype=torch.float32, device=q.device)
    z_snap = torch.empty((B, H, n, Dk), dtype=torch.float32, device=q.device)
    s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    z_final = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    kind = KIND_GATED if alpha is not None else KIND_FORWARD
    ws = _workspace(workspace_size(kind, B, H, N, Dk, Dv, code), q.device, workspace)
    rc = lib().linattn_forward_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(s_init),
                                         _ptr(z_init), _ptr(s_final), _ptr(z_final),
                                         ctypes.cast(parr, ctypes.c_void_p), n, _ptr(s_snap), _ptr(z_snap), B, H, N,
                                         Dk, Dv, code, phi, float(eps), _ptr(ws), _ws_bytes(ws), _stream(q))
    _check(rc, "linattn_forward_snapshots")
    return o, s_snap, z_snap, s_final, z_final


def linattn_forward_noncausal(q, k, v, *, eps=1e-6, phi=PHI_ELU1, want_state=True, out=None, workspace=None):
    """Non-causal form -> (o, s, z) with the global state s [B, H, Dk, Dv], z [B, H, Dk]."""
    (B, H, N, Dk, Dv, code), specs = _qkv_specs(q, k, v)
    _validate(specs + [(out, "out", (B, H, N, Dv), q.dtype)])
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    s = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_state else None
    z = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device) if want_state else None
    ws = _workspace(workspace_size(KIND_NONCAUSAL, B, H, N, Dk, Dv, code), q.device, workspace)
    rc = lib().linattn_forward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s), _ptr(z), B, H, N, Dk, Dv,
                                         code, phi, float(eps), _ptr(ws), _ws_bytes(ws), _stream(q))
    _check(rc, "linattn_forward_noncausal")
    return o, s, z


def _decode_specs(q, k, v, s, z, alpha, out, state_dtype):
    B, H, Dk = _dims(q, "q", 3)
    Dv = _dims(v, "v", 3)[2]
    code = _dtype_code(q)
    specs = [(q, "q", (B, H, Dk), None), (k, "k", (B, H, Dk), q.dtype), (v, "v", (B, H, Dv), q.dtype),
             (s, "s", (B, H, Dk, Dv), state_dtype), (z, "z", (B, H, Dk), state_dtype),
             (alpha, "alpha", (B, H), torch.float32), (out, "out", (B, H, Dv), q.dtype)]
    if s is None or z is None:
        raise ValueError("s and z are required")
    _validate(specs)
    return B, H, Dk, Dv, code


def linattn_decode_step(q, k, v, s, z, alpha=None, *, eps=1e-6, phi=PHI_ELU1, out=None):
    """One token per (b, h): q, k [B, H, Dk], v [B, H, Dv]; s, z updated in place; returns o [B, H, Dv]."""
    B, H, Dk, Dv, code = _decode_specs(q, k, v, s, z, alpha, out, torch.float32)
    o = out if out is not None else torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    rc = lib().linattn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(z), _ptr(alpha), _ptr(o), B, H, Dk,
                                   Dv, code, phi, float(eps), _stream(q))
    _check(rc, "linattn_decode_step")
    return o


_STATE_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}


def linattn_decode_step_lowp(q, k, v, s, z, alpha=None, *, eps=1e-6, phi=PHI_ELU1, out=None):
    """linattn_decode_step with S, z stored as float32, bfloat16 or float8_e4m3fn (their dtype decides)."""
    if not isinstance(s, torch.Tensor) or s.dtype not in _STATE_CODES:
        raise TypeError("s must be float32, bfloat16 or float8_e4m3fn")
    B, H, Dk, Dv, code = _decode_specs(q, k, v, s, z, alpha, out, s.dtype)
    o = out if out is not None else torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    rc = lib().linattn_decode_step_lowp(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(z), _STATE_CODES[s.dtype],
                                        _ptr(alpha), _ptr(o), B, H, Dk, Dv, code, phi, float(eps), _stream(q))
    _check(rc, "linattn_decode_step_lowp")
    return o


def linattn_abi_version() -> int:
    return int(lib().linattn_abi_version())


def linattn_status_string(rc: int) -> str:
    return lib().linattn_status_string(rc).decode()


def linattn_profile_enable(on: bool):
    _check(lib().linattn_profile_enable(1 if on else 0), "linattn_profile_enable")


def linattn_profile_read(max_entries: int = 32):
    """{kernel name: (launches, total_ms)} of the launches since profiling was enabled."""
    names = (ctypes.c_char_p * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_int * max_entries)()
    n = lib().linattn_profile_read(ctypes.cast(names, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p),
                                   ctypes.cast(cnt, ctypes.c_void_p), max_entries)
    if n < 0:
        _check(n, "linattn_profile_read")
    return {names[i].decode(): (cnt[i], ms[i]) for i in range(min(n, max_entries))}
