"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything is launched.

Every call here is built to fail validation (or is pure host arithmetic), so
no kernel is ever launched on the fake pointers used below.
"""
import ctypes
import os
import re

import pytest

from linear_attention_phi_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

OK, EINVAL, ESHAPE, EDTYPE, EWORKSPACE, ELAUNCH = 0, -1, -2, -3, -4, -5
P = ctypes.c_void_p
FAKE = [P((i + 1) << 36) for i in range(12)]  # far apart, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(linattn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    # LINATTN_ABI_LIB: another build of the same library (the sanitizer run
    # in test_sanitizers.py points it at a host-instrumented one)
    path = os.environ.get("LINATTN_ABI_LIB")
    if not path:
        return b.lib()
    h = ctypes.CDLL(path)
    for name, (args, res) in b.SIGNATURES.items():
        getattr(h, name).argtypes = args
        getattr(h, name).restype = res
    return h


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    # and the binding declares a signature for each of them
    assert set(names) == set(b.SIGNATURES)


def test_abi_version_matches_header(L):
    m = re.search(r"#define LINATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert L.linattn_abi_version() == int(m.group(1))


def test_status_strings(L):
    for rc in (OK, EINVAL, ESHAPE, EDTYPE, EWORKSPACE, ELAUNCH):
        assert L.linattn_status_string(rc)
    assert L.linattn_status_string(-99) == b"unknown status"


def test_workspace_size_is_host_arithmetic(L):
    ws = L.linattn_workspace_size
    # one segment per head, no prefix needed
    assert ws(0, 1, 1, 64, 16, 16, 0) == 0
    assert ws(0, 256, 32, 64, 128, 128, 1) == 0
    # long sequence on few heads: 16 segments of 2 state cells each, plus the
    # state at the end of the sequence (snapshots near the end start from it)
    cell = (128 * 128 + 128) * 4
    n = ws(0, 1, 16, 131072, 128, 128, 1)
    assert n >= 16 * (16 * 2 + 1) * cell
    assert ws(1, 1, 16, 131072, 128, 128, 1) > n  # plus the gate products
    assert ws(2, 1, 1, 64, 16, 16, 0) > 0          # non-causal always needs the total
    # the backward keeps forward (with the column sums of V) and reverse
    # segment states, and dd of every token
    assert ws(3, 1, 16, 131072, 128, 128, 1) >= 16 * 2 * (16 * 2) * cell + 16 * 131072 * 4
    assert ws(3, 1, 1, 64, 64, 64, 1) >= 64 * 4  # dd even with one segment
    # the training forward keeps its segment states with the column sums of V
    assert ws(4, 1, 16, 131072, 128, 128, 1) >= 16 * (16 - 1) * 2 * (cell + 128 * 4)
    assert ws(4, 1, 1, 64, 64, 64, 1) == 0       # one segment: nothing to keep
    # invalid arguments -> 0
    assert ws(5, 1, 1, 64, 16, 16, 0) == 0
    assert ws(0, 0, 1, 64, 16, 16, 0) == 0
    assert ws(0, 1, 1, 64, 48, 16, 0) == 0
    assert ws(0, 1, 1, 64, 16, 16, 7) == 0


def fwd(L, q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], si=None, zi=None, sf=None, zf=None, B=1, H=1, N=64, Dk=16,
        Dv=16, dtype=0, phi=0, eps=1e-6, ws=None, wsb=0):
    return L.linattn_forward(q, k, v, o, si, zi, sf, zf, B, H, N, Dk, Dv, dtype, phi, eps, ws, wsb, None)


def test_forward_rejects_bad_arguments(L):
    assert fwd(L, q=None) == EINVAL
    assert fwd(L, o=None) == EINVAL
    assert fwd(L, B=0) == EINVAL
    assert fwd(L, H=-1) == EINVAL
    assert fwd(L, N=0) == EINVAL
    assert fwd(L, eps=-1.0) == EINVAL
    assert fwd(L, eps=float("nan")) == EINVAL
    assert fwd(L, eps=float("inf")) == EINVAL
    assert fwd(L, Dk=48) == ESHAPE
    assert fwd(L, Dv=256) == ESHAPE
    assert fwd(L, Dk=8) == ESHAPE
    assert fwd(L, dtype=2) == EDTYPE
    assert fwd(L, phi=5) == EDTYPE
    assert fwd(L, si=FAKE[4]) == EINVAL           # s_init without z_init
    assert fwd(L, zf=FAKE[5]) == EINVAL           # z_final without s_final
    assert fwd(L, o=P(FAKE[0].value + 64)) == EINVAL  # o overlaps q
    assert fwd(L, o=FAKE[2]) == EINVAL            # o is v
    # a long sequence needs a workspace: none, or one byte short
    need = L.linattn_workspace_size(0, 1, 2, 8192, 64, 64, 1)
    assert need > 0
    assert fwd(L, B=1, H=2, N=8192, Dk=64, Dv=64, dtype=1) == EWORKSPACE
    assert fwd(L, B=1, H=2, N=8192, Dk=64, Dv=64, dtype=1, ws=FAKE[6], wsb=need - 1) == EWORKSPACE


def test_gated_requires_alpha(L):
    rc = L.linattn_forward_gated(FAKE[0], FAKE[1], FAKE[2], None, FAKE[3], None, None, None, None, 1, 1, 64, 16, 16,
                                 0, 0, 1e-6, None, 0, None)
    assert rc == EINVAL
    need = L.linattn_workspace_size(1, 1, 1, 1 << 16, 32, 32, 1)
    rc = L.linattn_forward_gated(FAKE[0], FAKE[1], FAKE[2], FAKE[4], FAKE[3], None, None, None, None, 1, 1, 1 << 16,
                                 32, 32, 1, 0, 1e-6, FAKE[5], need - 1, None)
    assert rc == EWORKSPACE


def test_noncausal_rejects_bad_arguments(L):
    f = L.linattn_forward_noncausal
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, 1, 1, 64, 16, 16, 0, 0, 1e-6, FAKE[5], 1 << 20,
             None) == EINVAL
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], None, None, 1, 1, 64, 16, 16, 0, 0, 1e-6, None, 0, None) == EWORKSPACE
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], None, None, 1, 1, 64, 24, 16, 0, 0, 1e-6, FAKE[5], 1 << 20,
             None) == ESHAPE


def test_decode_rejects_bad_arguments(L):
    f = L.linattn_decode_step
    assert f(FAKE[0], FAKE[1], FAKE[2], None, FAKE[4], None, FAKE[5], 2, 2, 16, 16, 0, 0, 1e-6, None) == EINVAL
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, FAKE[5], 0, 2, 16, 16, 0, 0, 1e-6, None) == EINVAL
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, FAKE[5], 2, 2, 16, 12, 0, 0, 1e-6, None) == ESHAPE
    assert f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, FAKE[5], 2, 2, 16, 16, 3, 0, 1e-6, None) == EDTYPE
    # s and z overlap (z inside s)
    s = FAKE[3]
    assert f(FAKE[0], FAKE[1], FAKE[2], s, P(s.value + 256), None, FAKE[5], 2, 2, 16, 16, 0, 0, 1e-6,
             None) == EINVAL
    # o inside s
    assert f(FAKE[0], FAKE[1], FAKE[2], s, FAKE[4], None, P(s.value + 64), 2, 2, 16, 16, 0, 0, 1e-6, None) == EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(TypeError):
        b.linattn_forward(x, x, x)


def _shape_cases():
    """Calls through the binding, each with one caller tensor of a wrong size.

    The tensors live on the CPU: the binding checks every shape before it
    looks at devices, so each call must raise ValueError and nothing can be
    launched.
    """
    import torch
    B, H, N, D = 1, 2, 8, 16
    bf = torch.bfloat16
    q = torch.zeros(B, H, N, D, dtype=bf)
    s = torch.zeros(B, H, D, D)
    z = torch.zeros(B, H, D)
    a = torch.ones(B, H, N)
    bad_s, bad_z = torch.zeros(B, H, D, D + 1), torch.zeros(B, H, D + 1)
    bad_o = torch.zeros(B, H, N - 1, D, dtype=bf)
    qd = torch.zeros(B, H, D, dtype=bf)
    return {
        "forward s_init": lambda: b.linattn_forward(q, q, q, bad_s, z),
        "forward z_init": lambda: b.linattn_forward(q, q, q, s, bad_z),
        "forward out": lambda: b.linattn_forward(q, q, q, out=bad_o),
        "forward s_final": lambda: b.linattn_forward(q, q, q, s_final=bad_s, z_final=z),
        "forward z_final": lambda: b.linattn_forward(q, q, q, s_final=s, z_final=bad_z),
        "forward k": lambda: b.linattn_forward(q, bad_o, q),
        "forward v": lambda: b.linattn_forward(q, q, bad_o),
        "gated alpha": lambda: b.linattn_forward_gated(q, q, q, torch.ones(B, H, N + 1)),
        "planned out": lambda: b.linattn_forward_planned(q, q, q, 2, 1, out=bad_o),
        "train s_init": lambda: b.linattn_forward_train(q, q, q, bad_s, z),
        "backward den": lambda: b.linattn_backward(q, q, q, torch.zeros(B, H, N + 1), q),
        "backward dout": lambda: b.linattn_backward(q, q, q, a, bad_o),
        "backward z_init": lambda: b.linattn_backward(q, q, q, a, q, s, bad_z),
        "backward dq": lambda: b.linattn_backward(q, q, q, a, q, out=(bad_o, q, q)),
        "backward dk": lambda: b.linattn_backward(q, q, q, a, q, out=(q, bad_o, q)),
        "backward dv": lambda: b.linattn_backward(q, q, q, a, q, out=(q, q, bad_o)),
        "snapshots s_init": lambda: b.linattn_forward_snapshots(q, q, q, [0], s_init=bad_s, z_init=z),
        "snapshots alpha": lambda: b.linattn_forward_snapshots(q, q, q, [0], alpha=torch.ones(B, H + 1, N)),
        "snapshots position": lambda: b.linattn_forward_snapshots(q, q, q, [N]),
        "delta s_init": lambda: b.linattn_forward_delta(q, q, q, s_init=bad_s),
        "delta out": lambda: b.linattn_forward_delta(q, q, q, out=bad_o),
        "delta beta": lambda: b.linattn_forward_delta(q, q, q, beta=torch.ones(B, H, N - 1)),
        "noncausal out": lambda: b.linattn_forward_noncausal(q, q, q, out=bad_o),
        "decode v": lambda: b.linattn_decode_step(qd, qd, torch.zeros(B, H + 1, D, dtype=bf), s, z),
        "decode s": lambda: b.linattn_decode_step(qd, qd, qd, bad_s, z),
        "decode out": lambda: b.linattn_decode_step(qd, qd, qd, s, z, out=torch.zeros(B, H, D + 1, dtype=bf)),
        "decode alpha": lambda: b.linattn_decode_step(qd, qd, qd, s, z, torch.ones(B, H, 1)),
        "decode lowp z": lambda: b.linattn_decode_step_lowp(qd, qd, qd, s.to(bf), torch.zeros(B, H, D + 1, dtype=bf)),
    }


@pytest.mark.parametrize("case", sorted(_shape_cases()))
def test_binding_checks_every_tensor_shape_before_any_launch(case):
    with pytest.raises(ValueError):
        _shape_cases()[case]()


def test_binding_checks_dtype_before_device():
    import torch
    q = torch.zeros(1, 1, 8, 16, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="float32"):
        b.linattn_forward(q, q, q, torch.zeros(1, 1, 16, 16, dtype=torch.float64), torch.zeros(1, 1, 16))
    with pytest.raises(TypeError, match="bfloat16"):
        b.linattn_forward(q, q.float(), q)


def planned(L, segments=2, subsegments=1, B=1, H=1, N=8192, Dk=64, Dv=64, dtype=1, ws=None, wsb=0, alpha=None):
    return L.linattn_forward_planned(FAKE[0], FAKE[1], FAKE[2], alpha, FAKE[3], None, None, None, None, B, H, N,
                                     Dk, Dv, dtype, 0, 1e-6, segments, subsegments, ws, wsb, None)


def test_planned_forward_rejects_bad_arguments_and_sizes_its_workspace(L):
    assert planned(L, segments=0) == EINVAL
    assert planned(L, subsegments=0) == EINVAL
    assert planned(L, Dk=48) == ESHAPE
    wsp = L.linattn_workspace_size_planned
    cell = (64 * 64 + 64) * 4
    # one segment: no prefix, no workspace, even for a long sequence
    assert wsp(0, 1, 1, 8192, 64, 64, 1, 1, 1) == 0
    # 8192 tokens = 128 chunks: 4 segments of 32 chunks, 2 parts each, plus the end state
    assert wsp(0, 1, 1, 8192, 64, 64, 1, 4, 2) >= (4 * 2 + 1) * cell
    # a part count that does not divide the segment's chunks falls to a divisor: 32 chunks, 3 -> 2
    assert wsp(0, 1, 1, 8192, 64, 64, 1, 4, 3) == wsp(0, 1, 1, 8192, 64, 64, 1, 4, 2)
    # more segments than chunks: one chunk each
    assert wsp(0, 1, 1, 8192, 64, 64, 1, 1000, 1) == wsp(0, 1, 1, 8192, 64, 64, 1, 128, 1)
    assert wsp(1, 1, 1, 8192, 64, 64, 1, 4, 2) > wsp(0, 1, 1, 8192, 64, 64, 1, 4, 2)  # gate products
    assert wsp(2, 1, 1, 8192, 64, 64, 1, 4, 2) == 0    # kinds other than the causal forward
    assert wsp(0, 1, 1, 8192, 64, 64, 1, 0, 1) == 0
    need = wsp(0, 1, 1, 8192, 64, 64, 1, 4, 2)
    assert planned(L, segments=4, subsegments=2, ws=FAKE[6], wsb=need - 1) == EWORKSPACE
    # a split whose state cells of one (b, h) reach 1 GiB (the prefix addresses them through one
    # buffer descriptor): 2^21 tokens of 128-dim heads in one segment per chunk (32768 cells of 66 KB,
    # 2.2 GB) or per two chunks (1.1 GB)
    big = 1 << 21
    assert wsp(0, 1, 1, big, 128, 128, 1, big // 64, 1) == 0
    assert wsp(0, 1, 1, big, 128, 128, 1, big // 128, 1) == 0
    assert planned(L, segments=big // 64, N=big, Dk=128, Dv=128, ws=FAKE[6], wsb=1 << 40) == ESHAPE
    # below the limit (4096 cells, 273 MB) the call is sized normally
    assert wsp(0, 1, 1, big, 128, 128, 1, big // 512, 1) > 0


def train(L, q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], den=FAKE[4], B=1, H=1, N=64, Dk=64, Dv=64, dtype=1,
          phi=0, eps=1e-6, ws=None, wsb=0):
    return L.linattn_forward_train(q, k, v, o, den, None, None, None, None, B, H, N, Dk, Dv, dtype, phi, eps, ws,
                                   wsb, None)


def bwd(L, q=FAKE[0], k=FAKE[1], v=FAKE[2], den=FAKE[4], g=FAKE[5], dq=FAKE[6], dk=FAKE[7], dv=FAKE[8], si=None,
        zi=None, B=1, H=1, N=64, Dk=64, Dv=64, dtype=1, phi=0, eps=1e-6, ws=FAKE[10], wsb=1 << 20, saved=None):
    return L.linattn_backward(q, k, v, den, saved, g, dq, dk, dv, si, zi, B, H, N, Dk, Dv, dtype, phi, eps, ws, wsb,
                              None)


def test_training_forward_and_backward_reject_bad_arguments(L):
    # chunked bf16 path only
    assert train(L, dtype=0) == EDTYPE
    assert train(L, Dk=32) == ESHAPE
    assert train(L, Dv=16) == ESHAPE
    for name in ("o", "den"):
        assert train(L, **{name: None}) == EINVAL, name
    assert train(L, den=FAKE[0]) == EINVAL  # den overlaps q
    assert train(L, den=FAKE[3]) == EINVAL  # den overlaps o
    assert bwd(L, dtype=0) == EDTYPE
    assert bwd(L, Dk=32, Dv=128) == ESHAPE
    for name in ("q", "k", "v", "den", "g", "dq", "dk", "dv"):
        assert bwd(L, **{name: None}) == EINVAL, name
    assert bwd(L, eps=-1.0) == EINVAL
    assert bwd(L, ws=None, wsb=0) == EWORKSPACE  # dd lives in the workspace
    assert bwd(L, si=FAKE[9]) == EINVAL           # s_init without z_init
    assert bwd(L, dq=FAKE[0]) == EINVAL            # output overlaps an input
    assert bwd(L, dk=FAKE[6]) == EINVAL            # outputs overlap each other
    assert bwd(L, B=0) == EINVAL
    assert bwd(L, phi=5) == EDTYPE
    # 8192 tokens on one head run many segments: the saved states are read, and
    # must not overlap an output or the workspace
    need = L.linattn_workspace_size(3, 1, 1, 8192, 64, 64, 1)
    assert L.linattn_workspace_size(4, 1, 1, 8192, 64, 64, 1) > 0
    assert bwd(L, N=8192, wsb=need, saved=FAKE[6]) == EINVAL
    assert bwd(L, N=8192, wsb=need, saved=FAKE[10]) == EINVAL
    # long sequence on one head: segment states needed, workspace missing
    assert bwd(L, N=131072) == EWORKSPACE
    need = L.linattn_workspace_size(3, 1, 1, 131072, 64, 64, 1)
    assert bwd(L, N=131072, ws=FAKE[10], wsb=need - 1) == EWORKSPACE


def delta(L, q=FAKE[0], k=FAKE[1], v=FAKE[2], alpha=None, beta=None, o=FAKE[3], si=None, sf=None, B=1, H=1, N=64,
          Dk=64, Dv=64, dtype=1, phi=0):
    return L.linattn_forward_delta(q, k, v, alpha, beta, o, si, sf, B, H, N, Dk, Dv, dtype, phi, None)


def test_delta_rejects_bad_arguments(L):
    assert delta(L, dtype=0) == EDTYPE
    assert delta(L, Dk=32) == ESHAPE
    assert delta(L, phi=7) == EDTYPE
    for name in ("q", "k", "v", "o"):
        assert delta(L, **{name: None}) == EINVAL, name
    assert delta(L, o=FAKE[0]) == EINVAL    # o overlaps q
    assert delta(L, sf=FAKE[3]) == EINVAL   # s_final overlaps o
    assert delta(L, N=0) == EINVAL
    assert delta(L, alpha=FAKE[3]) == EINVAL  # gates overlap o


def snaps(L, positions=(0, 5), n=None, ss=FAKE[6], zs=FAKE[7], N=64, Dk=64, Dv=64, dtype=1, alpha=None):
    arr = (ctypes.c_int * max(1, len(positions)))(*positions) if positions is not None else None
    n = len(positions) if n is None and positions is not None else (n or 0)
    return L.linattn_forward_snapshots(FAKE[0], FAKE[1], FAKE[2], alpha, FAKE[3], None, None, None, None,
                                       ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, n, ss, zs,
                                       1, 1, N, Dk, Dv, dtype, 0, 1e-6, None, 0, None)


def test_snapshots_reject_bad_arguments(L):
    assert snaps(L, dtype=0) == EDTYPE
    assert snaps(L, Dk=16, Dv=16) == ESHAPE
    assert snaps(L, positions=None) == EINVAL
    assert snaps(L, positions=[0], n=0) == EINVAL
    assert snaps(L, positions=list(range(257)), N=1000) == EINVAL  # more than LINATTN_MAX_SNAPSHOTS
    assert snaps(L, positions=[64]) == EINVAL                       # past the end (N = 64)
    assert snaps(L, positions=[-1]) == EINVAL
    assert snaps(L, ss=None) == EINVAL
    assert snaps(L, ss=FAKE[0]) == EINVAL                           # s_snap overlaps q
    assert snaps(L, zs=FAKE[6]) == EINVAL                           # z_snap overlaps s_snap


def noalloc(L, q=FAKE[0], k=FAKE[1], v=FAKE[2], o=FAKE[3], si=None, zi=None, sf=None, zf=None, B=1, H=1, N=64,
            Dk=16, Dv=16, dtype=0, phi=0, eps=1e-6):
    return L.linattn_forward_noalloc(q, k, v, o, si, zi, sf, zf, B, H, N, Dk, Dv, dtype, phi, eps, None)


def test_noalloc_forward_rejects_bad_arguments_and_oversized_calls(L):
    assert noalloc(L, q=None) == EINVAL
    assert noalloc(L, o=None) == EINVAL
    assert noalloc(L, B=0) == EINVAL
    assert noalloc(L, Dk=48) == ESHAPE
    assert noalloc(L, dtype=5) == EDTYPE
    assert noalloc(L, si=FAKE[4]) == EINVAL            # s_init without z_init
    assert noalloc(L, o=FAKE[0]) == EINVAL             # o overlaps q
    # fp32 over 65536 tokens of one 128-dim head runs 1024 segments: 64.6 MiB of
    # segment states, more than the fixed 48 MiB scratch -> refused, nothing runs
    need = L.linattn_workspace_size(0, 1, 1, 65536, 128, 128, 0)
    assert need > 48 << 20
    assert noalloc(L, N=65536, Dk=128, Dv=128) == EWORKSPACE
    # the long bf16 workload fits
    assert L.linattn_workspace_size(0, 1, 16, 131072, 128, 128, 1) <= 48 << 20
    assert b.NOALLOC_SCRATCH_BYTES == 48 << 20
    m = re.search(r"#define LINATTN_NOALLOC_SCRATCH_BYTES (\d+)u", open(HEADER).read())
    assert int(m.group(1)) == b.NOALLOC_SCRATCH_BYTES


def test_noalloc_binding_refuses_oversized_calls_before_any_launch():
    import torch
    q = torch.zeros(1, 1, 65536, 128)
    with pytest.raises(ValueError, match="scratch"):
        b.linattn_forward_noalloc(q, q, q)
