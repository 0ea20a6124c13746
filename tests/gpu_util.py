"""Helpers for GPU parity tests: move tensors to float64 numpy, compare with the
stated tolerances, and lay global tensors out into rings with the LIBRARY's
positions (the oracle always uses its own positions for the reference)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances.
#   fp32 inputs: norm-wise relative 1e-4 on out and lse (and gradients).
#   bf16 inputs: 2e-2 max-abs on out, 1e-3 max-abs on lse; gradients
#   2e-2 * max(1, max|ref|) (bf16 P and dS inside the kernels).
F32_REL = 1e-4
BF16_OUT_ABS = 2e-2
BF16_LSE_ABS = 1e-3
BF16_GRAD_REL = 2e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def _finite_match(got, ref, what):
    gi, ri = ~np.isfinite(got), ~np.isfinite(ref)
    assert np.array_equal(gi, ri), f"{what}: non-finite pattern differs ({gi.sum()} vs {ri.sum()})"
    if gi.any():
        assert np.array_equal(got[gi], ref[gi]), f"{what}: infinities differ"
    return ~ri


def check_out(got, ref, dtype_is_bf16: bool, what="out"):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    m = _finite_match(got, ref, what)
    if not m.any():
        return 0.0
    err = float(np.max(np.abs(got[m] - ref[m])))
    if dtype_is_bf16:
        tol = BF16_OUT_ABS
    else:
        tol = F32_REL * max(float(np.max(np.abs(ref[m]))), 1e-30)
    assert err <= tol, f"{what}: max abs err {err:.3e} > tol {tol:.3e}"
    return err


def check_lse(got, ref, dtype_is_bf16: bool, what="lse"):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    m = _finite_match(got, ref, what)
    if not m.any():
        return 0.0
    err = float(np.max(np.abs(got[m] - ref[m])))
    tol = BF16_LSE_ABS if dtype_is_bf16 else F32_REL * max(float(np.max(np.abs(ref[m]))), 1e-30)
    assert err <= tol, f"{what}: max abs err {err:.3e} > tol {tol:.3e}"
    return err


def check_grad(got, ref, dtype_is_bf16: bool, what="grad"):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = BF16_GRAD_REL * max(1.0, mx) if dtype_is_bf16 else F32_REL * max(mx, 1e-30)
    assert err <= tol, f"{what}: max abs err {err:.3e} > tol {tol:.3e} (max|ref| {mx:.3e})"
    return err


def ring_from_global(x, layout: str, world: int, cu_seqlens=None):
    """[b, S, h, d] -> [world, b, S/world, h, d] using the library's positions
    (the per-sequence layouts need cu_seqlens)."""
    import torch
    import exact_long_context_ra_amd as ra
    S = x.shape[1]
    cu = cu_seqlens if layout.endswith("_varlen") else None
    idx = [torch.from_numpy(ra.layout_positions(layout, S, world, r, cu)).to(x.device) for r in range(world)]
    return torch.stack([x.index_select(1, i) for i in idx]).contiguous(), idx


def varlen_cu_multiple(S: int, unit: int):
    """cu_seqlens of packed lengths that are multiples of `unit` (as the
    per-sequence layouts need): single units, an empty sequence, runs that
    straddle tiles, and the rest of S as the last sequence."""
    import synth
    lengths = [unit, 0, 8 * unit, unit, 17 * unit, 33 * unit, unit]
    rest = S - sum(lengths)
    assert rest > 0 and rest % unit == 0
    return synth.cu_seqlens(lengths + [rest])


def varlen_cu_many(S: int, unit: int, n: int = 21):
    """cu_seqlens of n packed sequences (more than one grouped launch holds),
    lengths multiples of `unit` from 1 to 11 units, the rest of S last."""
    import synth
    lengths = [unit * (1 + (i * 7) % 11) for i in range(n - 1)]
    rest = S - sum(lengths)
    assert rest > 0 and rest % unit == 0
    return synth.cu_seqlens(lengths + [rest])


def oracle_rows_fwd_bwd(q, k, v, dout, qpos, kpos, causal, cu_seqlens=None, block=64, workers=None):
    """The oracle's forward and backward for many query rows, run on row blocks
    in a thread pool (numpy and BLAS release the GIL; BLAS is held to one thread
    per block).  q/dout [b, Lq, h, d] (rows at positions qpos), k/v [b, Lk, h, d]
    at SORTED positions kpos.  Each block is given only the keys it can see (a
    contiguous range of kpos: none past its last row when causal, none before the
    start of its first row's sequence with cu_seqlens); the keys left out are
    masked for every row of the block, so the results are those of the whole key
    set.  Returns out, lse, dq of the rows and the rows' contributions dk, dv to
    every key (float64)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    assert np.all(np.diff(kpos) > 0), "kpos must be sorted"
    B, Lq, H, Dh = q.shape
    out = np.zeros((B, Lq, H, v.shape[3]))
    lse = np.full((B, H, Lq), -np.inf)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)

    def key_range(rows):
        lo, hi = 0, kpos.size
        pmin, pmax = int(qpos[rows].min()), int(qpos[rows].max())
        if causal:
            hi = int(np.searchsorted(kpos, pmax, side="right"))
        if cu is not None:
            s0 = int(cu[np.searchsorted(cu, pmin, side="right") - 1])
            lo = int(np.searchsorted(kpos, s0, side="left"))
            if not causal:
                e1 = int(cu[np.searchsorted(cu, pmax, side="right")])
                hi = int(np.searchsorted(kpos, e1, side="left"))
        return lo, max(lo, hi)

    def work(i0):
        rows = np.arange(i0, min(Lq, i0 + block))
        lo, hi = key_range(rows)
        kb, vb, kp = k[:, lo:hi], v[:, lo:hi], kpos[lo:hi]
        o, l = oracle.attention(q[:, rows], kb, vb, qpos[rows], kp, causal, cu_seqlens)
        gq, gk, gv = oracle.attention_backward(q[:, rows], kb, vb, o, l, dout[:, rows], qpos[rows], kp, causal,
                                               cu_seqlens)
        return rows, lo, hi, o, l, gq, gk, gv

    nw = workers or min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=nw) as ex:
        for rows, lo, hi, o, l, gq, gk, gv in ex.map(work, range(0, Lq, block)):
            out[:, rows] = o
            lse[:, :, rows] = l
            dq[:, rows] = gq
            dk[:, lo:hi] += gk
            dv[:, lo:hi] += gv
    return out, lse, dq, dk, dv
