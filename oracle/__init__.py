"""fp64 CPU oracle for causal linear attention with phi(x) = elu(x) + 1.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``linear_attention_phi_amd``) and neither imports the
other; both consume the same seeded inputs from ``linear_attention_phi_amd.synth``
(which holds no arithmetic of the method).

Three independent routes to the same quantities live here:

* ``forward`` / ``forward_gated`` / ``noncausal`` / ``decode_step`` call the
  plain per-token recurrence in ``linattn_oracle.c`` (fp64, one token at a
  time, OpenMP over (batch, head) pairs only); ``backward`` calls its adjoint.
* ``quadratic_forward`` (in ``quadratic.py``) is the masked N x N form written
  with NumPy, for tiny inputs.
* ``state_from_prefix`` sums the outer products with a library matrix product
  (the accumulation equals phi(K)^T V: "Linear Attention: accumulating KV into
  a fixed-size state", section "Adding to the same state in turn").

All inputs are taken as the exact stored values (fp32 or bf16 upcast to fp64).
parity pinned: every function here is checked in ``tests/test_oracle.py``
against the pages' worked examples, closed forms and the quadratic form.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .quadratic import quadratic_backward, quadratic_forward  # noqa: F401

PHI_ELU1 = 0
PHI_IDENTITY = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB = os.path.join(_HERE, "liblinattn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (portable x86-64 code, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # LINATTN_ORACLE_LIB points the pins at a deliberately broken build
            # (tests/test_oracle_mutants.py); normally unset.
            path = os.environ.get("LINATTN_ORACLE_LIB") or build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
            lib.oracle_forward.argtypes = [P] * 9 + [i64, i64, i32, i32, i32, f64, i32]
            lib.oracle_forward.restype = i32
            lib.oracle_noncausal.argtypes = [P] * 6 + [i64, i64, i32, i32, i32, f64, i32]
            lib.oracle_noncausal.restype = i32
            lib.oracle_decode_step.argtypes = [P] * 7 + [i64, i32, i32, i32, f64, i32]
            lib.oracle_decode_step.restype = i32
            lib.oracle_backward.argtypes = [P] * 12 + [i64, i64, i32, i32, i32, f64, i32]
            lib.oracle_backward.restype = i32
            lib.oracle_delta.argtypes = [P] * 8 + [i64, i64, i32, i32, i32, i32]
            lib.oracle_delta.restype = i32
            lib.oracle_decode_lowp.argtypes = [P] * 7 + [i64, i32, i32, i32, f64, i32]
            lib.oracle_decode_lowp.restype = i32
            lib.oracle_state_round.argtypes = [f64, i32]
            lib.oracle_state_round.restype = f64
            lib.oracle_phi.argtypes = [P, P, i64, i32]
            lib.oracle_phi.restype = None
            _lib = lib
    return _lib


def _threads(n_items: int) -> int:
    return max(1, min(n_items, os.cpu_count() or 1))


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a CPU torch tensor (e.g. bf16): upcast exactly
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def phi(x, mode: int = PHI_ELU1):
    x = _f64(np.asarray(x, dtype=np.float64))
    y = np.empty_like(x)
    _load().oracle_phi(_ptr(x), _ptr(y), x.size, mode)
    return y


def forward(q, k, v, s_init=None, z_init=None, *, alpha=None, eps=1e-6,
            phi_mode=PHI_ELU1, want_o=True, nthreads=None):
    """Causal forward over [B, H, N, D] inputs; returns (O, S_final, z_final) in fp64.

    ``alpha`` ([B, H, N]) turns on the per-token decay of S and z, applied
    before token t is added.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, H, N, Dk) and v.shape == (B, H, N, Dv)
    a = _f64(alpha)
    if a is not None:
        assert a.shape == (B, H, N)
    si, zi = _f64(s_init), _f64(z_init)
    if si is not None:
        assert si.shape == (B, H, Dk, Dv) and zi is not None and zi.shape == (B, H, Dk)
    o = np.empty((B, H, N, Dv)) if want_o else None
    s = np.empty((B, H, Dk, Dv))
    z = np.empty((B, H, Dk))
    rc = _load().oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(si), _ptr(zi),
                                _ptr(o), _ptr(s), _ptr(z), B * H, N, Dk, Dv, phi_mode,
                                float(eps), nthreads or _threads(B * H))
    if rc != 0:
        raise RuntimeError("oracle_forward failed")
    return o, s, z


def snapshots(q, k, v, positions, s_init=None, z_init=None, *, alpha=None, phi_mode=PHI_ELU1, nthreads=None):
    """The summary after each listed token, in fp64: (S_p, z_p) is the final state of the
    forward over tokens 0..p ("Linear Attention: what happens when you change the product
    order", section "What a summary can't do": restoring a summary needs a copy taken at that
    exact position).  Returns s [B, H, n, Dk, Dv], z [B, H, n, Dk].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    a = _f64(alpha)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    pos = [int(p) for p in positions]
    s = np.empty((B, H, len(pos), Dk, Dv))
    z = np.empty((B, H, len(pos), Dk))
    for i, p in enumerate(pos):
        assert 0 <= p < N
        _, s[:, :, i], z[:, :, i] = forward(q[:, :, :p + 1], k[:, :, :p + 1], v[:, :, :p + 1], s_init, z_init,
                                            alpha=None if a is None else a[:, :, :p + 1], phi_mode=phi_mode,
                                            want_o=False, nthreads=nthreads)
    return s, z


def delta(q, k, v, beta=None, s_init=None, *, alpha=None, phi_mode=PHI_ELU1, want_o=True, nthreads=None):
    """Delta-rule forward ("Linear Attention: what happens when you change the product order",
    section "The summary runs out of room"): per token, decay the summary by alpha (the gated
    form, Gated DeltaNet), read it with the unit key phi(k)/|phi(k)|, write beta times the
    difference to the value, read with phi(q).  alpha, beta [B, H, N] or None (ones).
    Returns (O, S_final) in fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, H, N, Dk) and v.shape == (B, H, N, Dv)
    b = _f64(beta)
    if b is not None:
        assert b.shape == (B, H, N)
    a = _f64(alpha)
    if a is not None:
        assert a.shape == (B, H, N)
    si = _f64(s_init)
    if si is not None:
        assert si.shape == (B, H, Dk, Dv)
    o = np.empty((B, H, N, Dv)) if want_o else None
    s = np.empty((B, H, Dk, Dv))
    rc = _load().oracle_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(si), _ptr(o), _ptr(s), B * H, N,
                              Dk, Dv, phi_mode, nthreads or _threads(B * H))
    if rc != 0:
        raise RuntimeError("oracle_delta failed")
    return o, s


def forward_gated(q, k, v, alpha, s_init=None, z_init=None, **kw):
    return forward(q, k, v, s_init, z_init, alpha=alpha, **kw)


def noncausal(q, k, v, *, eps=1e-6, phi_mode=PHI_ELU1, nthreads=None):
    """Non-causal form: one global (S, z) read by every query; returns (O, S, z)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    o = np.empty((B, H, N, Dv))
    s = np.empty((B, H, Dk, Dv))
    z = np.empty((B, H, Dk))
    rc = _load().oracle_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s), _ptr(z),
                                  B * H, N, Dk, Dv, phi_mode, float(eps),
                                  nthreads or _threads(B * H))
    if rc != 0:
        raise RuntimeError("oracle_noncausal failed")
    return o, s, z


def decode_step(q, k, v, s, z, *, alpha=None, eps=1e-6, phi_mode=PHI_ELU1, nthreads=None):
    """One token per (b, h): q, k [B, H, Dk], v [B, H, Dv], s [B, H, Dk, Dv], z [B, H, Dk].

    Returns (o, s_new, z_new); the inputs are not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = _f64(s).copy()
    z = _f64(z).copy()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    a = _f64(alpha)
    o = np.empty((B, H, Dv))
    rc = _load().oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(s), _ptr(z),
                                    _ptr(o), B * H, Dk, Dv, phi_mode, float(eps),
                                    nthreads or _threads(B * H))
    if rc != 0:
        raise RuntimeError("oracle_decode_step failed")
    return o, s, z


STATE_F32, STATE_BF16, STATE_FP8_E4M3 = 0, 1, 2


def state_round(x, state_dtype):
    """Elementwise rounding to a state storage type (bf16, OCP fp8 e4m3 with NaN past 448, or fp32)."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().oracle_state_round
    return np.vectorize(lambda t: f(float(t), state_dtype), otypes=[np.float64])(x)


def decode_lowp(q, k, v, s, z, state_dtype, *, alpha=None, eps=1e-6, phi_mode=PHI_ELU1):
    """One decode step with the state stored in a narrower type ("Linear Attention: what happens when
    you change the product order", section "What a summary can't do": a summary rewritten every token
    in low precision).  s, z hold stored values (float64 arrays); returns (o, s_new, z_new).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = _f64(s).copy()
    z = _f64(z).copy()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    a = _f64(alpha)
    o = np.empty((B, H, Dv))
    rc = _load().oracle_decode_lowp(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(s), _ptr(z), _ptr(o), B * H, Dk, Dv,
                                    phi_mode, float(eps), state_dtype)
    if rc != 0:
        raise RuntimeError("oracle_decode_lowp failed")
    return o, s, z


def backward(q, k, v, dout, s_init=None, z_init=None, *, alpha=None, eps=1e-6, phi_mode=PHI_ELU1,
             nthreads=None):
    """Gradients of a loss L through the causal forward, given dout = dL/dO.

    Returns (dq, dk, dv, ds_init, dz_init) in fp64; the gates ``alpha`` are
    constants.  The adjoint of the per-token recurrence in ``linattn_oracle.c``.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, H, N, Dk) and v.shape == (B, H, N, Dv) and dout.shape == (B, H, N, Dv)
    a = _f64(alpha)
    si, zi = _f64(s_init), _f64(z_init)
    dq = np.empty((B, H, N, Dk))
    dk = np.empty((B, H, N, Dk))
    dv = np.empty((B, H, N, Dv))
    ds = np.empty((B, H, Dk, Dv))
    dz = np.empty((B, H, Dk))
    rc = _load().oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(si), _ptr(zi), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds), _ptr(dz), B * H, N, Dk, Dv,
                                 phi_mode, float(eps), nthreads or _threads(B * H))
    if rc != 0:
        raise RuntimeError("oracle_backward failed")
    return dq, dk, dv, ds, dz


def state_from_prefix(k, v, phi_mode=PHI_ELU1):
    """(S, z) after a prefix, as one library contraction per head: S = phi(K)^T V, z = sum phi(k).

    k: [..., N, Dk], v: [..., N, Dv] -> S [..., Dk, Dv], z [..., Dk] in fp64.
    The accumulated outer products equal the single product phi(K)^T V
    ("Linear Attention: accumulating KV into a fixed-size state", section
    "Adding to the same state in turn").
    """
    k, v = _f64(k), _f64(v)
    fk = phi(k, phi_mode)
    s = np.matmul(np.swapaxes(fk, -1, -2), v)
    z = fk.sum(axis=-2)
    return s, z
