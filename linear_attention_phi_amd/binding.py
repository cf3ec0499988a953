"""Thin ctypes binding of ``include/linattn.h`` for torch tensors.

Argument marshalling only: shapes and dtypes are checked, device pointers and
the current HIP stream are handed to the C ABI, and every step of the method
runs in the HIP library.  There is no fallback: if ``liblinattn.so`` is
missing, or a call returns an error status, a RuntimeError is raised.
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
KIND_FORWARD, KIND_GATED, KIND_NONCAUSAL, KIND_BACKWARD = 0, 1, 2, 3

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
    "linattn_forward_train": ([_P] * 9 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_backward": ([_P] * 10 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_decode_step_lowp": ([_P] * 5 + [_I] + [_P] * 2 + [_I] * 6 + [_F, _P], _I),
    "linattn_forward_delta": ([_P] * 8 + [_I] * 7 + [_P], _I),
    "linattn_forward_snapshots": ([_P] * 10 + [_I] + [_P] * 2 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_forward_noncausal": ([_P] * 6 + [_I] * 7 + [_F, _P, _SZ, _P], _I),
    "linattn_decode_step": ([_P] * 7 + [_I] * 6 + [_F, _P], _I),
    "linattn_workspace_size": ([_I] * 7, _SZ),
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


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def workspace_size(kind, B, H, N, Dk, Dv, dtype_code) -> int:
    return int(lib().linattn_workspace_size(kind, B, H, N, Dk, Dv, dtype_code))


def _workspace(kind, B, H, N, Dk, Dv, code, device, workspace):
    need = workspace_size(kind, B, H, N, Dk, Dv, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


def linattn_forward(q, k, v, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, want_state=True,
                    out=None, s_final=None, z_final=None, workspace=None):
    """Causal forward.  q, k [B, H, N, Dk]; v [B, H, N, Dv] -> (o, s_final, z_final)."""
    return _forward(False, q, k, v, None, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace)


def linattn_forward_gated(q, k, v, alpha, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1,
                          want_state=True, out=None, s_final=None, z_final=None, workspace=None):
    """Gated causal forward with alpha [B, H, N] fp32 -> (o, s_final, z_final)."""
    return _forward(True, q, k, v, alpha, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace)


def _forward(gated, q, k, v, alpha, s_init, z_init, eps, phi, want_state, out, s_final, z_final, workspace):
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k, v shapes do not match")
    if gated:
        _dev(alpha, "alpha", torch.float32)
        if tuple(alpha.shape) != (B, H, N):
            raise ValueError("alpha must be [B, H, N]")
    if (s_init is None) != (z_init is None):
        raise ValueError("pass both s_init and z_init or neither")
    _dev(s_init, "s_init", torch.float32)
    _dev(z_init, "z_init", torch.float32)
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    _dev(o, "out", q.dtype)
    if want_state:
        s_final = s_final if s_final is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                   device=q.device)
        z_final = z_final if z_final is not None else torch.empty((B, H, Dk), dtype=torch.float32,
                                                                   device=q.device)
        _dev(s_final, "s_final", torch.float32)
        _dev(z_final, "z_final", torch.float32)
    else:
        s_final = z_final = None
    kind = KIND_GATED if gated else KIND_FORWARD
    ws, need = _workspace(kind, B, H, N, Dk, Dv, code, q.device, workspace)
    L = lib()
    if gated:
        rc = L.linattn_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(s_init), _ptr(z_init),
                                     _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps),
                                     _ptr(ws), ws.numel(), _stream(q))
    else:
        rc = L.linattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s_init), _ptr(z_init), _ptr(s_final),
                               _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws), ws.numel(),
                               _stream(q))
    _check(rc, "linattn_forward_gated" if gated else "linattn_forward")
    return o, s_final, z_final


def linattn_forward_train(q, k, v, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, workspace=None):
    """Causal forward that also keeps each token's denominator -> (o, den, s_final, z_final).

    bf16 with Dk, Dv in {64, 128}; den [B, H, N] fp32 feeds linattn_backward.
    """
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k, v shapes do not match")
    if (s_init is None) != (z_init is None):
        raise ValueError("pass both s_init and z_init or neither")
    _dev(s_init, "s_init", torch.float32)
    _dev(z_init, "z_init", torch.float32)
    o = torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    z_final = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    ws, _ = _workspace(KIND_FORWARD, B, H, N, Dk, Dv, code, q.device, workspace)
    rc = lib().linattn_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _ptr(s_init), _ptr(z_init),
                                     _ptr(s_final), _ptr(z_final), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws),
                                     ws.numel(), _stream(q))
    _check(rc, "linattn_forward_train")
    return o, den, s_final, z_final


def linattn_backward(q, k, v, den, dout, s_init=None, z_init=None, *, eps=1e-6, phi=PHI_ELU1, out=None,
                     workspace=None):
    """Gradients of a loss through the causal forward, given dout = dL/dO -> (dq, dk, dv).

    den is the output of linattn_forward_train on the same q, k, v (and
    initial state, eps, phi).  ``out`` may pass preallocated (dq, dk, dv).
    """
    _dev(q, "q")
    code = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _dev(t, name, q.dtype)
    _dev(den, "den", torch.float32)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if (tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape) != (B, H, N, Dv) or tuple(dout.shape) != (B, H, N, Dv)
            or tuple(den.shape) != (B, H, N)):
        raise ValueError("q, k, v, den, dout shapes do not match")
    if (s_init is None) != (z_init is None):
        raise ValueError("pass both s_init and z_init or neither")
    _dev(s_init, "s_init", torch.float32)
    _dev(z_init, "z_init", torch.float32)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _dev(dq, "dq", q.dtype)
    _dev(dk, "dk", q.dtype)
    _dev(dv, "dv", q.dtype)
    ws, _ = _workspace(KIND_BACKWARD, B, H, N, Dk, Dv, code, q.device, workspace)
    rc = lib().linattn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(den), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(s_init), _ptr(z_init), B, H, N, Dk, Dv, code, phi, float(eps), _ptr(ws),
                                ws.numel(), _stream(q))
    _check(rc, "linattn_backward")
    return dq, dk, dv


def linattn_forward_delta(q, k, v, beta=None, s_init=None, *, alpha=None, phi=PHI_ELU1, want_state=True,
                          out=None):
    """Delta rule: decay the summary by alpha (gated form), read it with the unit key
    phi(k)/|phi(k)|, write beta times the difference, o = S^T phi(q).  alpha, beta [B, H, N]
    fp32 or None (ones) -> (o, s_final or None).  bf16 with Dk, Dv in {64, 128}.
    """
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k, v shapes do not match")
    for name, t in (("beta", beta), ("alpha", alpha)):
        _dev(t, name, torch.float32)
        if t is not None and tuple(t.shape) != (B, H, N):
            raise ValueError(f"{name} must be [B, H, N]")
    _dev(s_init, "s_init", torch.float32)
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
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k, v shapes do not match")
    if (s_init is None) != (z_init is None):
        raise ValueError("pass both s_init and z_init or neither")
    _dev(s_init, "s_init", torch.float32)
    _dev(z_init, "z_init", torch.float32)
    _dev(alpha, "alpha", torch.float32)
    if alpha is not None and tuple(alpha.shape) != (B, H, N):
        raise ValueError("alpha must be [B, H, N]")
    pos = [int(p) for p in positions]
    n = len(pos)
    if not 1 <= n <= MAX_SNAPSHOTS:
        raise ValueError(f"1 to {MAX_SNAPSHOTS} positions")
    parr = (ctypes.c_int * n)(*pos)
    o = torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    s_snap = torch.empty((B, H, n, Dk, Dv), dtype=torch.float32, device=q.device)
    z_snap = torch.empty((B, H, n, Dk), dtype=torch.float32, device=q.device)
    s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    z_final = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device)
    kind = KIND_GATED if alpha is not None else KIND_FORWARD
    ws, _ = _workspace(kind, B, H, N, Dk, Dv, code, q.device, workspace)
    rc = lib().linattn_forward_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(s_init),
                                         _ptr(z_init), _ptr(s_final), _ptr(z_final),
                                         ctypes.cast(parr, ctypes.c_void_p), n, _ptr(s_snap), _ptr(z_snap), B, H, N,
                                         Dk, Dv, code, phi, float(eps), _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "linattn_forward_snapshots")
    return o, s_snap, z_snap, s_final, z_final


def linattn_forward_noncausal(q, k, v, *, eps=1e-6, phi=PHI_ELU1, want_state=True, out=None, workspace=None):
    """Non-causal form -> (o, s, z) with the global state s [B, H, Dk, Dv], z [B, H, Dk]."""
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, Dk) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k, v shapes do not match")
    o = out if out is not None else torch.empty((B, H, N, Dv), dtype=q.dtype, device=q.device)
    _dev(o, "out", q.dtype)
    s = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_state else None
    z = torch.empty((B, H, Dk), dtype=torch.float32, device=q.device) if want_state else None
    ws, need = _workspace(KIND_NONCAUSAL, B, H, N, Dk, Dv, code, q.device, workspace)
    rc = lib().linattn_forward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s), _ptr(z), B, H, N, Dk, Dv,
                                         code, phi, float(eps), _ptr(ws), ws.numel(), _stream(q))
    _check(rc, "linattn_forward_noncausal")
    return o, s, z


def linattn_decode_step(q, k, v, s, z, alpha=None, *, eps=1e-6, phi=PHI_ELU1, out=None):
    """One token per (b, h): q, k [B, H, Dk], v [B, H, Dv]; s, z updated in place; returns o [B, H, Dv]."""
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(s, "s", torch.float32)
    _dev(z, "z", torch.float32)
    if tuple(s.shape) != (B, H, Dk, Dv) or tuple(z.shape) != (B, H, Dk) or tuple(k.shape) != (B, H, Dk):
        raise ValueError("decode shapes do not match")
    if alpha is not None:
        _dev(alpha, "alpha", torch.float32)
        if tuple(alpha.shape) != (B, H):
            raise ValueError("alpha must be [B, H]")
    o = out if out is not None else torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(o, "out", q.dtype)
    rc = lib().linattn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(z), _ptr(alpha), _ptr(o), B, H, Dk,
                                   Dv, code, phi, float(eps), _stream(q))
    _check(rc, "linattn_decode_step")
    return o


_STATE_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}


def linattn_decode_step_lowp(q, k, v, s, z, alpha=None, *, eps=1e-6, phi=PHI_ELU1, out=None):
    """linattn_decode_step with S, z stored as float32, bfloat16 or float8_e4m3fn (their dtype decides)."""
    _dev(q, "q")
    code = _dtype_code(q)
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if s.dtype not in _STATE_CODES or z.dtype != s.dtype:
        raise TypeError("s and z must share one of float32, bfloat16, float8_e4m3fn")
    _dev(s, "s", s.dtype)
    _dev(z, "z", s.dtype)
    if tuple(s.shape) != (B, H, Dk, Dv) or tuple(z.shape) != (B, H, Dk) or tuple(k.shape) != (B, H, Dk):
        raise ValueError("decode shapes do not match")
    if alpha is not None:
        _dev(alpha, "alpha", torch.float32)
        if tuple(alpha.shape) != (B, H):
            raise ValueError("alpha must be [B, H]")
    o = out if out is not None else torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(o, "out", q.dtype)
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
