"""Throughput of causal linear attention (phi = elu + 1) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-paths]

One step is one causal forward over the long-context workload (B=1, H=16,
N=131072, Dk=Dv=128, bf16 in and out, fp32 state): the segment-state pass, the
prefix over segments and the chunked output pass, with inputs resident in HBM.
Prints ONE JSON line: tokens/s (B*N per step), the roofline fraction of the
dominant kernel (timed with HIP events recorded by the library around each of
its launches), the fp64 oracle timed on a bounded sample on the host cores,
and, under "paths", the decode step, the gated forward and the non-causal form
on their own workloads.

Also: ``--copy-calibration`` runs only a plain device copy of a known size
(for scaling the FETCH_SIZE / WRITE_SIZE counters), ``--path`` picks a single
workload to run (profiling runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_phi_amd import binding as la  # noqa: E402
from linear_attention_phi_amd import roofline as rf  # noqa: E402
from linear_attention_phi_amd import synth  # noqa: E402

METRIC = "causal linear-attn fwd Mtokens/s at N=128K,D=128; % of MFMA/HBM roofline"
HEADLINE = "long_n131072_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_phi_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# After an idle spell the MI355X's power management lets the first few
# milliseconds of a bandwidth-bound load run fast, then throttles hard (a
# 0.63 ms step takes up to 0.93 ms) and settles over roughly 30-40 ms.  The
# warm-up therefore runs W steps and at least SETTLE_S seconds of steps, so the
# timed steps see the sustained clock.
SETTLE_S = 0.1


def warm(fn, warmup):
    """Run the untimed warm-up; returns the number of steps it took."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-5)
    n = max(warmup, int(SETTLE_S / est) + 1)
    for _ in range(n - 2):
        fn()
    torch.cuda.synchronize()
    return n


def timed(fn, steps, warmup, stream):
    """Average ms per step over exactly `steps` steps, after the warm-up."""
    warm(fn, warmup)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def kernel_times(fn, steps):
    """Average device ms per launch of each library kernel, from the library's own HIP events."""
    la.linattn_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    rec = la.linattn_profile_read()
    la.linattn_profile_enable(False)
    return {k: {"launches": n, "avg_ms": ms / n} for k, (n, ms) in rec.items()}


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter runs, if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel, {}).get(workload)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


# ------------------------------------------------------------------ workloads
def forward_case(name, dev):
    w = synth.WORKLOADS[name]
    q, k, v = (x.to(dev) for x in synth.qkv(w))
    a = synth.alpha(w).to(dev) if w.gated else None
    kind = la.KIND_GATED if w.gated else la.KIND_FORWARD
    ws = torch.empty(max(1, la.workspace_size(kind, w.B, w.H, w.N, w.Dk, w.Dv, la.BF16)), dtype=torch.uint8,
                     device=dev)
    o = torch.empty((w.B, w.H, w.N, w.Dv), dtype=w.dtype, device=dev)
    s = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    z = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    if w.gated:
        def fn():
            la.linattn_forward_gated(q, k, v, a, out=o, s_final=s, z_final=z, workspace=ws)
    else:
        def fn():
            la.linattn_forward(q, k, v, out=o, s_final=s, z_final=z, workspace=ws)
    nbytes = rf.forward_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2, gated=w.gated)
    return w, fn, nbytes, (q, k, v, a)


def backward_case(name, dev, inputs=None):
    """Backward over a forward workload: den from the training forward (untimed), dO seeded N(0, 1)."""
    w = synth.WORKLOADS[name]
    q, k, v = inputs if inputs is not None else (x.to(dev) for x in synth.qkv(w))
    g = synth.dout(w).to(dev)
    _, den, _, _ = la.linattn_forward_train(q, k, v)
    ws = torch.empty(la.workspace_size(la.KIND_BACKWARD, w.B, w.H, w.N, w.Dk, w.Dv, la.BF16), dtype=torch.uint8,
                     device=dev)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    def fn():
        la.linattn_backward(q, k, v, den, g, out=out, workspace=ws)
    return w, fn, rf.backward_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2)


SNAP_POSITIONS = "8 prefix-cache points at 16384 m - 1 (m = 1..8) and the last 8 tokens"


def snapshot_positions(N):
    return sorted({16384 * m - 1 for m in range(1, 9) if 16384 * m - 1 < N} | {N - 1 - i for i in range(8)})


def snapshots_case(name, dev, inputs=None):
    """Causal forward that also returns the state after snapshot_positions(N)."""
    w = synth.WORKLOADS[name]
    q, k, v = inputs if inputs is not None else (x.to(dev) for x in synth.qkv(w))
    pos = snapshot_positions(w.N)
    ws = torch.empty(la.workspace_size(la.KIND_FORWARD, w.B, w.H, w.N, w.Dk, w.Dv, la.BF16), dtype=torch.uint8,
                     device=dev)

    def fn():
        la.linattn_forward_snapshots(q, k, v, pos, workspace=ws)
    # the forward's bytes plus each snapshot's state written once
    nbytes = rf.forward_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2) + w.B * w.H * len(pos) * (w.Dk * w.Dv + w.Dk) * 4
    return w, fn, nbytes, pos


def delta_case(name, dev):
    """Delta rule over its own workload (beta absent: the full overwrite)."""
    w = synth.WORKLOADS[name]
    q, k, v = (x.to(dev) for x in synth.qkv(w))
    o = torch.empty((w.B, w.H, w.N, w.Dv), dtype=w.dtype, device=dev)

    def fn():
        la.linattn_forward_delta(q, k, v, out=o)
    return w, fn, rf.delta_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2)


def kernel_bytes(kernel, w):
    """Algorithmic bytes one launch of a library kernel moves on workload w (None if not a whole-pass kernel)."""
    if kernel == "delta_bf16":
        return rf.delta_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2)
    if kernel.startswith("bwd_"):
        return rf.backward_kernel_bytes(kernel, w.B, w.H, w.N, w.Dk, w.Dv, 2)
    if kernel.startswith("fwd_out_bf16"):
        return rf.forward_bytes(w.B, w.H, w.N, w.Dk, w.Dv, 2, gated=w.gated)
    if kernel == "decode_step":
        return rf.decode_bytes(w.B, w.H, w.Dk, w.Dv, 2)
    if kernel in ("seg_state_bf16", "noncausal_apply_bf16"):
        # non-causal: the state pass reads every K and V row once; the apply
        # pass reads Q and writes O once
        return w.B * w.H * w.N * (w.Dk + w.Dv) * 2
    return None


def kernel_flops(kernel, w, path_flops):
    """MFMA-level flops of one launch, where the kernel does the path's contractions."""
    if kernel.startswith("fwd_out"):
        return path_flops
    if kernel.startswith("bwd_"):
        return rf.backward_kernel_flops(kernel, w.B, w.H, w.N, w.Dk, w.Dv)
    if kernel == "delta_bf16":
        return rf.delta_flops(w.B, w.H, w.N, w.Dk, w.Dv)
    return None


def noncausal_case(name, dev, inputs=None):
    w = synth.WORKLOADS[name]
    q, k, v = inputs if inputs is not None else (x.to(dev) for x in synth.qkv(w))
    ws = torch.empty(la.workspace_size(la.KIND_NONCAUSAL, w.B, w.H, w.N, w.Dk, w.Dv, la.BF16), dtype=torch.uint8,
                     device=dev)
    o = torch.empty((w.B, w.H, w.N, w.Dv), dtype=w.dtype, device=dev)

    def fn():
        la.linattn_forward_noncausal(q, k, v, want_state=False, out=o, workspace=ws)
    # Q, K, V read once, O written once (the global state stays on chip / in workspace)
    nbytes = w.B * w.H * w.N * (2 * w.Dk + 2 * w.Dv) * 2
    return w, fn, nbytes


def decode_state(dev):
    """Decode workload: the state after a 2048-token seeded prefix, built by the library's own forward."""
    w = synth.WORKLOADS["decode_b256h32_d128"]
    s = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    z = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    for b in range(w.B):
        kp, vp = decode_prefix_gpu(w, b, dev)
        # the prefix's queries do not enter the state; keys stand in for them
        la.linattn_forward(kp, kp, vp, s_final=s[b:b + 1], z_final=z[b:b + 1])
    q, k, v = (x.to(dev) for x in synth.decode_token(w))
    return w, s, z, q, k, v


def decode_case(dev):
    w, s, z, q, k, v = decode_state(dev)
    o = torch.empty((w.B, w.H, w.Dv), dtype=w.dtype, device=dev)
    s0, z0 = s.clone(), z.clone()

    def fn():
        la.linattn_decode_step(q, k, v, s, z, out=o)

    def reset():
        s.copy_(s0)
        z.copy_(z0)
    nbytes = rf.decode_bytes(w.B, w.H, w.Dk, w.Dv, 2)
    return w, fn, nbytes, reset


def decode_lowp_case(dev, state_dtype):
    """The decode workload with the state stored in a narrower type (the prefix state rounded once)."""
    w, s32, z32, q, k, v = decode_state(dev)
    s0, z0 = s32.to(state_dtype), z32.to(state_dtype)
    s, z = s0.clone(), z0.clone()
    o = torch.empty((w.B, w.H, w.Dv), dtype=w.dtype, device=dev)

    def fn():
        la.linattn_decode_step_lowp(q, k, v, s, z, out=o)

    def reset():
        s.copy_(s0)
        z.copy_(z0)
    nbytes = rf.decode_bytes(w.B, w.H, w.Dk, w.Dv, 2, state_bytes=s0.element_size())
    return w, fn, nbytes, reset


def decode_prefix_gpu(w, b, dev):
    k, v = synth.decode_prefix(w, b)
    return k.unsqueeze(0).to(dev), v.unsqueeze(0).to(dev)


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, q, k, v, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the workload: all heads, the first n tokens."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1, w.B * w.H))
    n = 256
    while True:
        qs, ks, vs = (x[:, :, :n] for x in (q, k, v))
        t0 = time.perf_counter()
        oracle.forward(qs, ks, vs, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or n >= w.N:
            break
        n = min(w.N, int(n * max(2.0, min(16.0, budget_s / 2 / max(dt, 1e-3)))))
    tokens = w.B * n
    return {"value": tokens / dt / 1e6, "unit": "Mtokens/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.B * w.H} heads, first {n} of {w.N} tokens, fp64 recurrence (OpenMP over heads), "
                      f"{dt:.1f} s"}


# ------------------------------------------------------------------ main
def roofline_entry(kernel, avg_ms, nbytes, workload, flops=None):
    """nbytes: algorithmic bytes of ONE launch of this kernel."""
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    peak = rf.HBM_BYTES_PER_S / 1e9
    tr = stored_traffic(kernel, workload)
    out = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
           "frac": round(achieved / peak, 4), "traffic": tr, "algorithmic_bytes": nbytes,
           "avg_ms": round(avg_ms, 4)}
    if flops is not None:
        out["mfma_tflops"] = round(flops / (avg_ms * 1e-3) / 1e12, 1)
        out["mfma_frac"] = round(flops / (avg_ms * 1e-3) / rf.MFMA_BF16_FLOPS, 4)
    return out


def copy_calibration(dev, steps):
    """A plain device copy of exactly 1 GiB, for scaling the byte counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paths", action="store_true")
    ap.add_argument("--path", choices=["forward", "gated", "decode", "decode_bf16_state", "noncausal", "backward",
                                       "snapshots", "delta"],
                    default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the method is built and timed on a single GPU only; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        copy_calibration(dev, args.steps)
        return

    if args.path in ("decode", "decode_bf16_state", "gated", "noncausal", "backward", "snapshots", "delta"):
        # single-path run (used for counter collection); prints its own line
        run_single_path(args, dev, stream)
        return

    log(f"[bench] building inputs for {HEADLINE}")
    w, fn, nbytes, (q, k, v, _) = forward_case(HEADLINE, dev)
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    ms = timed(fn, args.steps, args.warmup, stream)
    kt = kernel_times(fn, args.steps)
    dom = max(kt, key=lambda n: kt[n]["avg_ms"] * kt[n]["launches"])
    flops = rf.chunked_flops(w.B, w.H, w.N, w.Dk, w.Dv, 64)
    tokens = w.B * w.N
    value = tokens / (ms * 1e-3) / 1e6
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "Mtokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": HEADLINE, "B": w.B, "H": w.H, "N": w.N, "Dk": w.Dk, "Dv": w.Dv,
                   "inputs": "bf16 N(0,1)/sqrt(128) for q, k, v; fp32 state; eps 1e-6"},
        "roofline": roofline_entry(dom, kt[dom]["avg_ms"], kernel_bytes(dom, w), HEADLINE, flops),
        "path_roofline_frac": round(rf.hbm_time_s(nbytes) / (ms * 1e-3), 4),
        "kernels_ms": {n: round(e["avg_ms"], 4) for n, e in kt.items()},
    }
    log(f"[bench] forward {ms:.3f} ms/step, {value:.1f} Mtok/s")
    if not args.no_paths:
        result["paths"] = other_paths(args, dev, stream, (q, k, v))
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a sample of the same workload")
        result["cpu_baseline"] = cpu_baseline(w, *(x.cpu() for x in (q, k, v)))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def path_entry(w, fn, nbytes, stream, args, tokens, reset=None, flops=None, key=None, kernel_nbytes=None):
    ms = timed(fn, args.steps, args.warmup, stream)
    if reset:
        reset()
    kt = kernel_times(fn, args.steps)
    if reset:
        reset()
    dom = max(kt, key=lambda n: kt[n]["avg_ms"] * kt[n]["launches"])
    key = key or w.name
    return {"workload": key, "ms_per_step": round(ms, 4), "Mtokens_per_s": round(tokens / (ms * 1e-3) / 1e6, 3),
            "path_roofline_frac": round(rf.hbm_time_s(nbytes) / (ms * 1e-3), 4),
            "roofline": roofline_entry(dom, kt[dom]["avg_ms"], kernel_nbytes or kernel_bytes(dom, w), key,
                                       kernel_flops(dom, w, flops)),
            "kernels_ms": {n: round(e["avg_ms"], 4) for n, e in kt.items()}}


def other_paths(args, dev, stream, headline_inputs):
    out = {}
    log("[bench] gated forward")
    w, fn, nbytes, _ = forward_case("gated_b2h16_n16384_d128", dev)
    out["gated"] = path_entry(w, fn, nbytes, stream, args, w.B * w.N,
                              flops=rf.chunked_flops(w.B, w.H, w.N, w.Dk, w.Dv, 64))
    del fn
    log("[bench] decode step")
    w, fn, nbytes, reset = decode_case(dev)
    out["decode"] = path_entry(w, fn, nbytes, stream, args, w.B, reset=reset)
    out["decode"]["steps_per_s"] = round(1e3 / out["decode"]["ms_per_step"], 1)
    del fn
    log("[bench] decode step, bf16 state")
    w, fn, nbytes, reset = decode_lowp_case(dev, torch.bfloat16)
    out["decode_bf16_state"] = path_entry(w, fn, nbytes, stream, args, w.B, reset=reset, key="decode_bf16_state",
                                          kernel_nbytes=nbytes)
    out["decode_bf16_state"]["steps_per_s"] = round(1e3 / out["decode_bf16_state"]["ms_per_step"], 1)
    del fn
    log("[bench] non-causal form")
    w, fn, nbytes = noncausal_case(HEADLINE, dev, headline_inputs)
    out["noncausal"] = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="noncausal_" + w.name)
    del fn
    log("[bench] forward with state snapshots")
    w, fn, nbytes, pos = snapshots_case(HEADLINE, dev, headline_inputs)
    out["snapshots"] = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="snapshots_" + w.name)
    out["snapshots"]["positions"] = SNAP_POSITIONS
    del fn
    log("[bench] backward")
    w, fn, nbytes = backward_case(HEADLINE, dev, headline_inputs)
    out["backward"] = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="backward_" + w.name,
                                 flops=rf.backward_flops(w.B, w.H, w.N, w.Dk, w.Dv))
    del fn
    log("[bench] delta rule")
    w, fn, nbytes = delta_case("delta_b16h16_n4096_d128", dev)
    out["delta"] = path_entry(w, fn, nbytes, stream, args, w.B * w.N,
                              flops=rf.delta_flops(w.B, w.H, w.N, w.Dk, w.Dv))
    return out


def run_single_path(args, dev, stream):
    if args.path == "gated":
        w, fn, nbytes, _ = forward_case("gated_b2h16_n16384_d128", dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B * w.N)
    elif args.path == "decode":
        w, fn, nbytes, reset = decode_case(dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B, reset=reset)
    elif args.path == "decode_bf16_state":
        w, fn, nbytes, reset = decode_lowp_case(dev, torch.bfloat16)
        r = path_entry(w, fn, nbytes, stream, args, w.B, reset=reset, key="decode_bf16_state", kernel_nbytes=nbytes)
    elif args.path == "delta":
        w, fn, nbytes = delta_case("delta_b16h16_n4096_d128", dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B * w.N, flops=rf.delta_flops(w.B, w.H, w.N, w.Dk, w.Dv))
    elif args.path == "snapshots":
        w, fn, nbytes, _ = snapshots_case(HEADLINE, dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="snapshots_" + w.name)
    elif args.path == "backward":
        w, fn, nbytes = backward_case(HEADLINE, dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="backward_" + w.name,
                       flops=rf.backward_flops(w.B, w.H, w.N, w.Dk, w.Dv))
    else:
        w, fn, nbytes = noncausal_case(HEADLINE, dev)
        r = path_entry(w, fn, nbytes, stream, args, w.B * w.N, key="noncausal_" + w.name)
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
