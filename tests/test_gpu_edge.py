"""Degenerate sizes through the C ABI: a block with no keys (every row gets
(out, lse) = (0, -inf), the empty-set case of the definition), a block with no
queries, a backward step with no keys, and an empty sequence through the ring
entry points.  None of them may fail or touch memory outside its outputs."""
import math

import pytest

import synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu


def _ra():
    import exact_long_context_ra_amd as ra
    return ra


def _dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_block_fwd_without_keys(D, dt):
    import torch
    ra = _ra()
    log(f"block fwd lk=0 D={D} {dt}")
    B, H, lq = 2, 3, 77
    (q,) = synth.draw_normal([(B, lq, H, D)], _dtype(dt), seed=5, device="cpu")
    q = q.to(dev())
    k = torch.empty((B, 0, H, D), device=dev(), dtype=q.dtype)
    out = torch.full((B, lq, H, D), float("nan"), device=dev())
    lse = torch.full((B, H, lq), float("nan"), device=dev())
    ra.block_attn_fwd(q, k, k, ra.posmap([(10, 1, lq)]), ra.posmap([(0, 1, 0)]), seq_len=100, causal=True,
                      out_b=out, lse_b=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out)), "rows with no key must give out = 0"
    assert bool(torch.all(lse == -math.inf)), "rows with no key must give lse = -inf"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_block_calls_without_queries_or_keys(dt):
    import torch
    ra = _ra()
    log(f"block fwd lq=0 and bwd lk=0 {dt}")
    B, H, D, n = 1, 2, 128, 96
    q, k, v, do = synth.draw_normal([(B, n, H, D)] * 4, _dtype(dt), seed=6, device="cpu")
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    empty = torch.empty((B, 0, H, D), device=dev(), dtype=q.dtype)
    # no queries: nothing to write, nothing read
    out0, lse0 = ra.block_attn_fwd(empty, k, v, ra.posmap([(0, 1, 0)]), ra.posmap([(0, 1, n)]), seq_len=n,
                                   causal=True)
    assert out0.shape[1] == 0 and lse0.shape[2] == 0
    # no keys in a backward step: the accumulators keep their values
    out, lse = ra.block_attn_fwd(q, k, v, ra.posmap([(0, 1, n)]), ra.posmap([(0, 1, n)]), seq_len=n, causal=True)
    delta = ra.bwd_preprocess(out, do)
    dq = torch.randn((B, n, H, D), device=dev())
    dq0 = dq.clone()
    dk_e = torch.empty((B, 0, H, D), device=dev(), dtype=torch.float32)
    ra.block_attn_bwd(q, empty, empty, do, lse, delta, ra.posmap([(0, 1, n)]), ra.posmap([(0, 1, 0)]), dq, dk_e,
                      dk_e, seq_len=n, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0), "a backward step without keys must leave dq_acc unchanged"


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
def test_ring_empty_sequence(layout):
    import torch
    ra = _ra()
    log(f"ring S=0 {layout}")
    N, H, D = 4, 2, 128
    ql = torch.empty((1, 0, H, D), device=dev(), dtype=torch.bfloat16)
    ring = torch.empty((N, 1, 0, H, D), device=dev(), dtype=torch.bfloat16)
    out, lse, _ = ra.ring_fwd(layout, N, 1, ql, ring, ring, causal=True)
    dq, dk, dv = ra.ring_bwd(layout, N, 1, ql, ring, ring, out, lse, ql, causal=True)
    torch.cuda.synchronize()
    assert out.numel() == 0 and lse.numel() == 0 and dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0
