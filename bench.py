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

Besides the headline workload, the default run also times the other layouts
(the stripe share, the contiguous ring over all ranks, the packed varlen
stream over all slices through the ring and through the gathered-K/V share,
and the per-sequence zigzag / stripe layouts) with a few steps each, reported
compactly under "other_workloads"; and it samples the GPU clock under load.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zigzag]
       [--also LIST|none] [--no-cpu-baseline]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
METRIC = "attention TFLOP/s (causal-adjusted) fwd and fwd+bwd, % bf16 MFMA peak"

WORKLOADS = {
    # name: (layout, seq_len, world, ranks timed, varlen, gathered K/V)
    "zigzag": ("zigzag", 131072, 8, [0], False, False),
    "stripe": ("stripe", 262144, 8, [0], False, False),
    "contiguous": ("contiguous", 32768, 8, list(range(8)), False, False),
    "varlen": ("contiguous", 131072, 8, list(range(8)), True, False),
    # the same packed sequences, every rank's slice against the whole gathered
    # K/V in one block step (llama3-style share)
    "varlen_gathered": ("contiguous", 131072, 8, list(range(8)), True, True),
    # per-sequence layouts: the same packed sequences, each laid out on its own
    # (lengths rounded to multiples of 2N / N); rank 0 (zigzag: every rank equal)
    "zigzag_varlen": ("zigzag_varlen", 131072, 8, [0], True, False),
    "stripe_varlen": ("stripe_varlen", 131072, 8, [0], True, False),
    # a long context: one million tokens on 8 ranks, rank 0's zigzag share (131072
    # rows; its dS^T goes through the backward in key chunks within 32 GiB)
    "zigzag_1m": ("zigzag", 1048576, 8, [0], False, False),
}
DEFAULT_ALSO = "stripe,contiguous,varlen,varlen_gathered,zigzag_varlen,stripe_varlen,zigzag_1m"
# timed steps of a secondary workload at most (a zigzag_1m step takes about 4 s)
MAX_ALSO_STEPS = {"zigzag_1m": 2}
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
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = sorted({f"{i.get('internal_api')} ({i.get('user_api')})" for i in info})
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
        blas = []
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
        "os_cpu_count": os.cpu_count(),
        "blas": blas,
    }


class Workload:
    """Resident inputs, outputs and workspace of one workload, and its step functions."""

    def __init__(self, name, ra, synth, torch, dev):
        layout, S, N, ranks, varlen, gathered = WORKLOADS[name]
        self.name, self.layout, self.S, self.N, self.ranks = name, layout, S, N, ranks
        self.varlen, self.gathered = varlen, gathered
        self.ra, self.torch = ra, torch
        H, D = HEADS, HEAD_DIM
        L = S // N
        cu = None
        if varlen:
            lengths = synth.loguniform_lengths(S, 1024, 32768, seed=0)
            if layout.endswith("_varlen"):
                lengths = synth.round_lengths(lengths, 2 * N if layout == "zigzag_varlen" else N)
            cu = synth.cu_seqlens(lengths)
        self.cu = cu
        # host and device copies made once: a plain array would be copied to the
        # device (and the stream waited for) on every call
        self.cu_arg = ra.CuSeqlens(cu, dev) if cu is not None else None
        # Inputs: global Q, K, V, dO drawn on the GPU, laid out into the ring by the
        # library's positions; all resident before timing.
        q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=0, device=dev, with_dout=True)
        idx = [torch.from_numpy(ra.layout_positions(layout, S, N, r, _lcu(layout, cu))).to(dev) for r in range(N)]
        self.k_ring = torch.stack([k.index_select(1, i) for i in idx]).contiguous()
        self.v_ring = torch.stack([v.index_select(1, i) for i in idx]).contiguous()
        del k, v
        self.q_loc = {r: q.index_select(1, idx[r]).contiguous() for r in ranks}
        self.do_loc = {r: do.index_select(1, idx[r]).contiguous() for r in ranks}
        del q, do
        self.out = {r: torch.empty((1, L, H, D), device=dev, dtype=torch.float32) for r in ranks}
        self.lse = {r: torch.empty((1, H, L), device=dev, dtype=torch.float32) for r in ranks}
        self.dq = torch.empty((1, L, H, D), device=dev, dtype=torch.float32)
        self.dk_ring = torch.zeros(self.k_ring.shape, device=dev, dtype=torch.float32)
        self.dv_ring = torch.zeros(self.v_ring.shape, device=dev, dtype=torch.float32)
        if gathered:
            # contiguous layout: the rank-major ring is the global token order
            assert layout == "contiguous"
            self.k_all = self.k_ring.view(1, S, H, D)
            self.v_all = self.v_ring.view(1, S, H, D)
            self.dk_all = self.dk_ring.view(1, S, H, D)
            self.dv_all = self.dv_ring.view(1, S, H, D)
            nbytes = max(ra.gathered_workspace_bytes(layout, N, r, self.q_loc[ranks[0]], cu_seqlens=cu)
                         for r in ranks)
        else:
            nbytes = ra.ring_workspace_bytes(layout, N, self.q_loc[ranks[0]], cu_seqlens=cu)
        self.ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)
        self.pairs = {r: step_pairs(ra, layout, S, N, r, cu) for r in ranks}
        self.total_pairs = sum(sum(p) for p in self.pairs.values())
        self.fwd_flops = 4.0 * D * H * self.total_pairs
        self.fb_flops = 3.5 * self.fwd_flops

    def fwd(self):
        ra = self.ra
        for r in self.ranks:
            if self.gathered:
                ra.gathered_fwd(self.layout, self.N, r, self.q_loc[r], self.k_all, self.v_all, causal=True,
                                cu_seqlens=self.cu_arg, out=self.out[r], lse=self.lse[r])
            else:
                ra.ring_fwd(self.layout, self.N, r, self.q_loc[r], self.k_ring, self.v_ring, causal=True,
                            cu_seqlens=self.cu_arg, out=self.out[r], lse=self.lse[r])

    def step(self):
        ra = self.ra
        for r in self.ranks:
            if self.gathered:
                ra.gathered_fwd(self.layout, self.N, r, self.q_loc[r], self.k_all, self.v_all, causal=True,
                                cu_seqlens=self.cu_arg, out=self.out[r], lse=self.lse[r])
                ra.gathered_bwd(self.layout, self.N, r, self.q_loc[r], self.k_all, self.v_all, self.out[r],
                                self.lse[r], self.do_loc[r], causal=True, cu_seqlens=self.cu_arg, dq=self.dq,
                                dk_all=self.dk_all, dv_all=self.dv_all, workspace=self.ws)
            else:
                ra.ring_fwd(self.layout, self.N, r, self.q_loc[r], self.k_ring, self.v_ring, causal=True,
                            cu_seqlens=self.cu_arg, out=self.out[r], lse=self.lse[r])
                ra.ring_bwd(self.layout, self.N, r, self.q_loc[r], self.k_ring, self.v_ring, self.out[r],
                            self.lse[r], self.do_loc[r], causal=True, cu_seqlens=self.cu_arg, dq=self.dq,
                            dk_ring=self.dk_ring, dv_ring=self.dv_ring, workspace=self.ws)

    def describe(self):
        r0 = self.ranks
        many = len(r0) > 1
        return (f"{self.layout} causal {'gathered-K/V (llama3-style) ' if self.gathered else 'ring '}"
                f"share{'s' if many else ''} "
                f"{'(varlen, log-uniform lengths in [1024, 32768]) ' if self.varlen else ''}"
                f"{'(lengths rounded to whole layout chunks) ' if self.layout.endswith('_varlen') else ''}"
                f"fwd+bwd: seq {self.S}, ring of {self.N}, rank{'s' if many else ''} "
                f"{r0 if many else r0[0]}, {HEADS} heads, head_dim {HEAD_DIM}, batch 1")


def timed_steps(torch, fn, steps):
    """Per-step milliseconds of `steps` calls of fn, each bracketed by events on
    the current stream, with a synchronisation before and after the region."""
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def sample_gfx_clock(torch, fn, seconds=2.0):
    """Median GFX clock (MHz, mean over the XCDs) that amd-smi reports while fn()
    runs back to back for about `seconds`; None where amd-smi is unavailable."""
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                out = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                                     text=True, timeout=10).stdout
                data = json.loads(out[out.index("{"):])
                clk = data["gpu_data"][0]["clock"] if "gpu_data" in data else data[0]["clock"]
                vals = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)
                        and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]
                if vals:
                    samples.append(sum(vals) / len(vals))
            except Exception:
                return

    th = threading.Thread(target=sampler, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end or (th.is_alive() and not samples and time.perf_counter() < t_end + 10):
        fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    # drop the first sample (the GPU may still be ramping up)
    use = samples[1:] if len(samples) > 2 else samples
    return round(statistics.median(use), 1) if use else None


def secondary(name, ra, synth, torch, dev, steps, warmup):
    """Compact timing of one more workload (fwd and fwd+bwd, `steps` each)."""
    w = Workload(name, ra, synth, torch, dev)
    for _ in range(warmup):
        w.step()
    fb = timed_steps(torch, w.step, steps)
    fw = timed_steps(torch, w.fwd, steps)
    res = {
        "workload": w.describe(),
        "ranks": w.ranks,
        "visible_pairs_per_head": w.total_pairs,
        "steps": steps,
        "ms_per_step": round(sum(fb) / steps, 3),
        "median_ms": round(statistics.median(fb), 3),
        "min_ms": round(min(fb), 3),
        "tflops": round(w.fb_flops / (sum(fb) / steps / 1e3) / 1e12, 2),
        "ms_fwd": round(sum(fw) / steps, 3),
        "fwd_min_ms": round(min(fw), 3),
        "fwd_tflops": round(w.fwd_flops / (sum(fw) / steps / 1e3) / 1e12, 2),
    }
    res["pct_peak_fwd_bwd"] = round(100 * res["tflops"] / PEAK_BF16_TFLOPS, 2)
    res["pct_peak_fwd"] = round(100 * res["fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="zigzag", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated further workloads timed compactly after the headline ('none': skip)")
    ap.add_argument("--also-steps", type=int, default=3)
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the GPU clock under load")
    ap.add_argument("--no-ring-eff", action="store_true", help="skip the ring-efficiency block-step timing")
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
    w = Workload(args.workload, ra, synth, torch, dev)
    H, D = HEADS, HEAD_DIM
    print(f"bench: {args.workload} inputs resident", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, bracketed by synchronisations; per-launch
    # HIP events recorded by the library on the launch stream give each
    # kernel's average duration.
    with ra.kernel_timing(capacity=8192) as kt:
        step_ms = timed_steps(torch, w.step, args.steps)
    ms_step = sum(step_ms) / args.steps

    # The per-launch event records leave about 10 us between launches; the
    # same K steps without them, reported beside the headline for reference.
    plain_ms = timed_steps(torch, w.step, args.steps)
    ms_step_plain = sum(plain_ms) / args.steps

    # Forward alone (second timed region, same inputs).
    fwd_ms = timed_steps(torch, w.fwd, args.steps)
    ms_fwd = sum(fwd_ms) / args.steps

    # Ring efficiency: N x the time of a causal self-attention block step of one
    # local chunk (the rank's queries against its own keys), over the time of the
    # rank's whole ring forward.
    ring_eff = None
    if not args.no_ring_eff and not w.gathered and len(w.ranks) == 1 and not w.layout.endswith("_varlen"):
        r = w.ranks[0]
        qm = ra.layout_posmap(w.layout, w.S, w.N, r)
        ob = torch.empty_like(w.out[r])
        lb = torch.empty_like(w.lse[r])

        def diag():
            ra.block_attn_fwd(w.q_loc[r], w.k_ring[r], w.v_ring[r], qm, qm, seq_len=w.S, causal=True,
                              cu_seqlens=w.cu_arg, out_b=ob, lse_b=lb)

        diag()
        d_ms = timed_steps(torch, diag, max(3, args.steps))
        t_diag = sum(d_ms) / len(d_ms)
        ring_eff = {"value": round(w.N * t_diag / ms_fwd, 4), "block_ms": round(t_diag, 4), "ring_fwd_ms": round(ms_fwd, 4),
                    "definition": "N x time(causal block step of one local chunk against itself) / time(ring forward)"}

    gfx_mhz = None if args.no_clock else sample_gfx_clock(torch, w.step)

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
            f * D * H * w.total_pairs * args.steps)
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

    value = w.fb_flops / (ms_step / 1e3) / 1e12
    fwd_tflops = w.fwd_flops / (ms_fwd / 1e3) / 1e12
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
            "workload": w.describe(),
            "layout": w.layout, "seq_len": w.S, "world": w.N, "ranks": w.ranks, "heads": H, "head_dim": D,
            "batch": 1, "causal": True, "varlen": w.varlen, "gathered_kv": w.gathered,
        },
        "pct_peak_fwd_bwd": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "pct_peak_fwd": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "ms_fwd": round(ms_fwd, 3),
        "step_ms_median": round(statistics.median(step_ms), 3),
        "step_ms_min": round(min(step_ms), 3),
        "fwd_ms_median": round(statistics.median(fwd_ms), 3),
        "fwd_ms_min": round(min(fwd_ms), 3),
        "ms_per_step_without_launch_events": round(ms_step_plain, 3),
        "visible_pairs_per_head": w.total_pairs,
        "ring_efficiency_fwd": ring_eff,
        "gfx_clock_mhz_under_load": gfx_mhz,
        "kernels": {n: {"launches": a["launches"], "avg_ms": round(a["ms"] / max(1, a["launches"]), 4),
                        **({"tflops": round(a["flops"] / (a["ms"] / 1e3) / 1e12, 1)} if a["flops"] and a["ms"] else {})}
                    for n, a in per_kernel.items() if a["launches"]},
        "roofline": roofline,
        "cpu_baseline": None,
        "other_workloads": {},
    }
    headline = (w.layout, w.S, w.N, list(w.ranks), w.varlen, w.gathered)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    also = [] if args.also in ("", "none") else [a.strip() for a in args.also.split(",") if a.strip()]
    for name in also:
        if name not in WORKLOADS or WORKLOADS[name] == headline:
            continue
        print(f"bench: {name}", file=sys.stderr, flush=True)
        steps = max(1, min(args.also_steps, MAX_ALSO_STEPS.get(name, args.also_steps)))
        res["other_workloads"][name] = secondary(name, ra, synth, torch, dev, steps, 1)
    if not args.no_cpu_baseline:
        lay, S, N, ranks, _, _ = WORKLOADS[args.workload]
        cu = None
        if WORKLOADS[args.workload][4]:
            lengths = synth.loguniform_lengths(S, 1024, 32768, seed=0)
            if lay.endswith("_varlen"):
                lengths = synth.round_lengths(lengths, 2 * N if lay == "zigzag_varlen" else N)
            cu = synth.cu_seqlens(lengths)
        res["cpu_baseline"] = cpu_baseline(lay, S, N, ranks[0], cu, D)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
