"""Benchmark of the ring-attention per-device hot path on one MI355X.

A step is one pass of the whole hot path over the workload: the virtual-ring
forward (all ring steps with the fused lse merge) followed by the ring
backward of the same rank share.  Default workload: the zigzag causal share of
rank 0 in an 8-rank ring over a 131072-token sequence, 32 heads, head_dim 128,
bf16 inputs ~ N(0, 1).  Inputs are resident in HBM before timing starts.

Metric: causal-adjusted attention TFLOP/s, i.e. exact visible (query, key)
pairs x 4 * head_dim * heads for the forward and 2.5x that for the backward
(5 matrix products per pair instead of 2), divided by the measured time.
Peak: MI355X dense bf16 MFMA, 2516.6 TFLOP/s (256 CU x 4096 FLOP/clk x 2.4 GHz).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zigzag]
       [--no-cpu-baseline]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
METRIC = "attention TFLOP/s (causal-adjusted) fwd and fwd+bwd, % bf16 MFMA peak"

WORKLOADS = {
    # name: (layout, seq_len, world, ranks timed, varlen)
    "zigzag": ("zigzag", 131072, 8, [0], False),
    "stripe": ("stripe", 262144, 8, [0], False),
    "contiguous": ("contiguous", 32768, 8, list(range(8)), False),
    "varlen": ("contiguous", 131072, 8, list(range(8)), True),
    # per-sequence layouts: the same packed sequences, each laid out on its own
    # (lengths rounded to multiples of 2N / N); rank 0 (zigzag: every rank equal)
    "zigzag_varlen": ("zigzag_varlen", 131072, 8, [0], True),
    "stripe_varlen": ("stripe_varlen", 131072, 8, [0], True),
}
HEADS, HEAD_DIM = 32, 128


def profiled_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic.txt (rocprofv3
    FETCH_SIZE/WRITE_SIZE, copy-calibrated), or None when the kernels changed
    since the counters were taken (source hash mismatch) or none were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    src = os.path.join(ROOT, "exact_long_context_ra_amd", "csrc", "ra_kernels.hip")
    try:
        lines = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    rec = {ln[0]: ln[1:] for ln in lines}
    if rec.get("kernel_source_sha256", [None])[0] != cur or kernel not in rec:
        return None
    vals = dict(zip(rec[kernel][::2], rec[kernel][1::2]))
    return int(vals["fetch_bytes"]) + int(vals["write_bytes"])


def visible_pairs(qpos: np.ndarray, kpos: np.ndarray, cu) -> int:
    """Exact causal visible pairs of sorted positions (varlen: same sequence)."""
    kpos = np.sort(kpos)
    hi = np.searchsorted(kpos, qpos, side="right")  # keys with pos <= q
    if cu is None:
        return int(hi.sum())
    cu = np.asarray(cu, dtype=np.int64)
    start = cu[np.searchsorted(cu, qpos, side="right") - 1]
    lo = np.searchsorted(kpos, start, side="left")  # keys with pos < seq start
    return int((hi - lo).sum())


def _lcu(layout, cu):
    """cu_seqlens as the layout functions take it (only the per-sequence layouts use it)."""
    return cu if layout.endswith("_varlen") else None


def step_pairs(ra, layout, S, N, r, cu):
    qpos = ra.layout_positions(layout, S, N, r, _lcu(layout, cu))
    return [visible_pairs(qpos, ra.layout_positions(layout, S, N, (r - s) % N, _lcu(layout, cu)), cu)
            for s in range(N)]


def cpu_baseline(layout, S, N, r, cu, D, seed=123):
    """Time the float64 oracle (as it stands) on a bounded sample of the same
    workload: one head, every 3rd query row of the first timed rank's share,
    against all keys; forward + backward (about 10 s on 16 host cores)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    qpos = oracle.layout_positions(layout, S, N, r, _lcu(layout, cu))
    rows = qpos[::3]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, len(rows), 1, D))
    k = rng.standard_normal((1, S, 1, D))
    v = rng.standard_normal((1, S, 1, D))
    do = rng.standard_normal((1, len(rows), 1, D))
    kpos = np.arange(S)
    t0 = time.perf_counter()
    o, l = oracle.attention(q, k, v, rows, kpos, True, cu)
    oracle.attention_backward(q, k, v, o, l, do, rows, kpos, True, cu)
    dt = time.perf_counter() - t0
    pairs = oracle.count_pairs(rows, kpos, True, cu)
    flops = 3.5 * 4 * D * pairs
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle fwd+bwd, 1 of {HEADS} heads, every 3rd query row of rank {r}'s "
                   f"{layout} share ({len(rows)} rows x {S} keys, {pairs} visible pairs), {dt:.1f} s"),
        "seconds": dt,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="zigzag", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run one plain device copy of MIB MiB (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (the virtual ring runs every ring step on it); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_long_context_ra_amd as ra
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    layout, S, N, ranks, varlen = WORKLOADS[args.workload]
    H, D = HEADS, HEAD_DIM
    L = S // N
    cu = None
    if varlen:
        lengths = synth.loguniform_lengths(S, 1024, 32768, seed=0)
        if layout.endswith("_varlen"):
            lengths = synth.round_lengths(lengths, 2 * N if layout == "zigzag_varlen" else N)
        cu = synth.cu_seqlens(lengths)

    # Inputs: global Q, K, V, dO drawn on the GPU, laid out into the ring by the
    # library's positions; all resident before timing.
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=0, device=dev, with_dout=True)
    idx = [torch.from_numpy(ra.layout_positions(layout, S, N, r, _lcu(layout, cu))).to(dev) for r in range(N)]
    k_ring = torch.stack([k.index_select(1, i) for i in idx]).contiguous()
    v_ring = torch.stack([v.index_select(1, i) for i in idx]).contiguous()
    del k, v
    q_loc = {r: q.index_select(1, idx[r]).contiguous() for r in ranks}
    do_loc = {r: do.index_select(1, idx[r]).contiguous() for r in ranks}
    del q, do
    out = {r: torch.empty((1, L, H, D), device=dev, dtype=torch.float32) for r in ranks}
    lse = {r: torch.empty((1, H, L), device=dev, dtype=torch.float32) for r in ranks}
    dq = torch.empty((1, L, H, D), device=dev, dtype=torch.float32)
    dk_ring = torch.zeros(k_ring.shape, device=dev, dtype=torch.float32)
    dv_ring = torch.zeros(v_ring.shape, device=dev, dtype=torch.float32)
    ws = torch.empty(ra.ring_workspace_bytes(layout, N, q_loc[ranks[0]], cu_seqlens=cu), device=dev,
                     dtype=torch.uint8)

    pairs = {r: step_pairs(ra, layout, S, N, r, cu) for r in ranks}
    total_pairs = sum(sum(p) for p in pairs.values())
    fwd_flops = 4.0 * D * H * total_pairs
    fb_flops = 3.5 * fwd_flops

    def fwd():
        for r in ranks:
            ra.ring_fwd(layout, N, r, q_loc[r], k_ring, v_ring, causal=True, cu_seqlens=cu,
                        out=out[r], lse=lse[r])

    def step():
        for r in ranks:
            ra.ring_fwd(layout, N, r, q_loc[r], k_ring, v_ring, causal=True, cu_seqlens=cu,
                        out=out[r], lse=lse[r])
            ra.ring_bwd(layout, N, r, q_loc[r], k_ring, v_ring, out[r], lse[r], do_loc[r], causal=True,
                        cu_seqlens=cu, dq=dq, dk_ring=dk_ring, dv_ring=dv_ring, workspace=ws)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, bracketed by synchronisations; per-launch
    # HIP events recorded by the library on the launch stream give each
    # kernel's average duration.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ra.kernel_timing(capacity=8192) as kt:
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # The per-launch event records leave about 10 us between launches; the
    # same K steps without them, reported beside the headline for reference.
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step_plain = ev0.elapsed_time(ev1) / args.steps

    # Forward alone (second timed region, same inputs).
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        fwd()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_fwd = ev0.elapsed_time(ev1) / args.steps

    # Per-kernel algorithmic FLOPs: each launch of block_fwd / block_bwd covers
    # one ring step of one rank: pairs(step) x 4*D*H (fwd) or x 10*D*H (bwd).
    per_kernel = {}
    for name, _, ms in kt.launches:
        agg = per_kernel.setdefault(name, {"launches": 0, "ms": 0.0, "flops": 0.0})
        agg["launches"] += 1
        agg["ms"] += ms
    # Matrix-product FLOPs each kernel executes over the timed region, per
    # visible pair and head: forward QK^T + PV = 4*D; the dK/dV kernel
    # recomputes S and dP and forms dV, dK = 8*D; the dQ kernel either reads the
    # dS the dK/dV kernel stored and forms dQ = 2*D, or (small workspace)
    # recomputes S and dP as well = 6*D.  (The metric above counts the backward
    # as 10*D per pair, the five products of the textbook gradient.)
    per_pair = {"block_fwd": 4.0, "block_bwd_dkdv": 8.0, "block_bwd_dq_ds": 2.0, "block_bwd_dq": 6.0}
    for name, f in per_pair.items():
        per_kernel.setdefault(name, {"launches": 0, "ms": 0.0, "flops": 0.0})["flops"] = (
            f * D * H * total_pairs * args.steps)
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms"])
    dk = per_kernel[dom]
    if dom in per_pair and dk["ms"] > 0:
        achieved = dk["flops"] / (dk["ms"] / 1e3) / 1e12
        traffic = profiled_traffic(dom) if args.workload == "zigzag" else None
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": dom,
                    "avg_launch_ms": dk["ms"] / max(1, dk["launches"]), "launches": dk["launches"]}
    else:
        roofline = {"bound": "hbm", "achieved": None, "peak": 8000.0, "unit": "GB/s", "frac": None,
                    "traffic": None, "kernel": dom}

    value = fb_flops / (ms_step / 1e3) / 1e12
    fwd_tflops = fwd_flops / (ms_fwd / 1e3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16, seeded)",
        "config": {
            "workload": (f"{layout} causal ring share{'s' if len(ranks) > 1 else ''} "
                         f"{'(varlen, log-uniform lengths in [1024, 32768]) ' if varlen else ''}"
                         f"{'(lengths rounded to whole layout chunks) ' if layout.endswith('_varlen') else ''}"
                         f"fwd+bwd: seq {S}, ring of {N}, rank{'s' if len(ranks) > 1 else ''} "
                         f"{ranks if len(ranks) > 1 else ranks[0]}, {H} heads, head_dim {D}, batch 1"),
            "layout": layout, "seq_len": S, "world": N, "ranks": ranks, "heads": H, "head_dim": D,
            "batch": 1, "causal": True, "varlen": varlen,
        },
        "pct_peak_fwd_bwd": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "pct_peak_fwd": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "ms_fwd": round(ms_fwd, 3),
        "ms_per_step_without_launch_events": round(ms_step_plain, 3),
        "visible_pairs_per_head": total_pairs,
        "kernels": {n: {"launches": a["launches"], "avg_ms": round(a["ms"] / max(1, a["launches"]), 4),
                        **({"tflops": round(a["flops"] / (a["ms"] / 1e3) / 1e12, 1)} if a["flops"] and a["ms"] else {})}
                    for n, a in per_kernel.items() if a["launches"]},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(layout, S, N, ranks[0], cu, D)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
