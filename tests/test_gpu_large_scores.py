"""Parity at large and growing scores: queries carry a constant offset and keys
an offset that grows with their position, so the scores of a row rise by about
180 over the sequence.  A row's maximum then grows on nearly every key tile
(the running output is rescaled again and again), P reaches values near the
rescale threshold between rescales, and the ring's LSE merges combine blocks
whose lse differ by more than a hundred.  HIP block and ring paths against the
float64 oracle on the same inputs."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_grad, check_lse, check_out, dev, f64, log, ring_from_global

pytestmark = pytest.mark.gpu


def _inputs(B, S, H, D, dtype, seed):
    """q ~ N(0,1) + 2, k at global position j ~ N(0,1) + 8 j / S, v, dO ~ N(0,1),
    rounded to `dtype` (both sides use the rounded values)."""
    import torch
    q, k, v, do = synth.draw_normal([(B, S, H, D)] * 4, torch.float32, seed=seed, device="cpu")
    ramp = (8.0 * torch.arange(S, dtype=torch.float32) / S).view(1, S, 1, 1)
    q = q + 2.0
    k = k + ramp
    return tuple(x.to(dtype).to(dev()) for x in (q, k, v, do))


def _row_growth(q64, k64):
    """Growth of the last row's scores along the keys (natural-log units): the
    mean over the last 64 keys minus the mean over the first 64, head 0."""
    s = (q64[0, -1, 0] @ k64[0, :, 0].T) / np.sqrt(q64.shape[-1])
    return float(np.mean(s[-64:]) - np.mean(s[:64]))


def _dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_block_growing_scores(causal, D, dt):
    import torch
    import exact_long_context_ra_amd as ra
    S, H, B = 640, 2, 1
    log(f"block growing scores causal={causal} D={D} {dt}")
    q, k, v, do = _inputs(B, S, H, D, _dtype(dt), seed=41)
    pos = np.arange(S)
    qm = km = ra.posmap([(0, 1, S)])
    out, lse = ra.block_attn_fwd(q, k, v, qm, km, seq_len=S, causal=causal)
    delta = ra.bwd_preprocess(out, do)
    dq = torch.zeros((B, S, H, D), device=dev(), dtype=torch.float32)
    dk = torch.zeros_like(dq)
    dv = torch.zeros_like(dq)
    ra.block_attn_bwd(q, k, v, do, lse, delta, qm, km, dq, dk, dv, seq_len=S, causal=causal)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, causal, None)
    # the inputs do what they are for: a row's scores grow by far more than the
    # rescale threshold (2^8, 5.5 in natural-log units) along the keys
    assert _row_growth(q64, k64) > 50.0
    bf = dt == "bf16"
    check_out(f64(out), ro, bf, what="out")
    check_lse(f64(lse), rl, bf, what="lse")
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, causal, None)
    check_grad(f64(dq), gq, bf, what="dq")
    check_grad(f64(dk), gk, bf, what="dk")
    check_grad(f64(dv), gv, bf, what="dv")


@pytest.mark.parametrize("dt,store_ds", [("bf16", True), ("bf16", False), ("f32", True)],
                         ids=["bf16-ds", "bf16-recompute", "f32"])
def test_zigzag_ring_growing_scores(dt, store_ds):
    """Every rank of a zigzag ring of 4: per-rank out/lse and dQ, and the
    summed dK/dV, against full causal attention over the whole sequence."""
    import torch
    import exact_long_context_ra_amd as ra
    layout, S, N, H, D = "zigzag", 1024, 4, 2, 128
    log(f"zigzag ring growing scores {dt} store_ds={store_ds}")
    q, k, v, do = _inputs(1, S, H, D, _dtype(dt), seed=43)
    kr, idx = ring_from_global(k, layout, N)
    vr, _ = ring_from_global(v, layout, N)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True, None)
    assert _row_growth(q64, k64) > 50.0 and float(np.max(rl) - np.min(rl)) > 100.0
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, True, None)
    bf = dt == "bf16"
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=True,
                               dk_ring=dk_ring, dv_ring=dv_ring, store_ds=store_ds)
        torch.cuda.synchronize()
        opos = oracle.layout_positions(layout, S, N, r, None)
        assert np.array_equal(opos, idx[r].cpu().numpy())
        check_out(f64(out), ro[:, opos], bf, what=f"out r={r}")
        check_lse(f64(lse), rl[:, :, opos], bf, what=f"lse r={r}")
        check_grad(f64(dq), gq[:, opos], bf, what=f"dq r={r}")
    check_grad(f64(dk_ring), oracle.to_ring(gk, layout, N, None), bf, what="dk (all ranks)")
    check_grad(f64(dv_ring), oracle.to_ring(gv, layout, N, None), bf, what="dv (all ranks)")
