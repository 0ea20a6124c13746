"""The autograd / packed / varlen / gathered-K/V forms against the oracle.

These wrap the same C ABI: q/k/v of a whole sequence are laid out into an
N-rank virtual ring, every rank's share runs ra_ring_fwd / ra_ring_bwd, and
the results come back in global order with autograd gradients."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_grad, check_lse, check_out, dev, f64, log

pytestmark = pytest.mark.gpu


def _ra():
    import exact_long_context_ra_amd as ra
    return ra


def _dt(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@pytest.mark.parametrize("layout,S,N,dt,B", [("zigzag", 1024, 4, "bf16", 1), ("stripe", 768, 4, "f32", 1),
                                             ("contiguous", 512, 4, "bf16", 2)])
def test_ring_attn_func_autograd(layout, S, N, dt, B):
    import torch
    ra = _ra()
    log(f"ring_attn_func {layout} S={S} N={N} {dt} batch={B}")
    H, D = 2, 128
    q, k, v, do = synth.qkv(S, H, D, _dt(dt), seed=41, device="cpu", batch=B, with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    out, lse = ra.ring_attn_func(qg, kg, vg, layout=layout, world=N, causal=True, return_lse=True)
    out.backward(do)
    torch.cuda.synchronize()
    pos = np.arange(S)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), pos, pos, True)
    gq, gk, gv = oracle.attention_backward(f64(q), f64(k), f64(v), ro, rl, f64(do), pos, pos, True)
    bf = dt == "bf16"
    check_out(f64(out), ro, bf)
    check_lse(f64(lse), rl, bf)
    check_grad(f64(qg.grad), gq, bf, what="dq")
    check_grad(f64(kg.grad), gk, bf, what="dk")
    check_grad(f64(vg.grad), gv, bf, what="dv")


def test_packed_forms_match_unpacked():
    """kv- and qkv-packed inputs (strided views) give bitwise the same results."""
    import torch
    ra = _ra()
    log("packed forms")
    S, H, D, N = 1024, 2, 64, 4
    qkv = synth.draw_normal([(1, S, 3, H, D)], torch.bfloat16, seed=43, device="cpu")[0].to(dev())
    q, k, v = (qkv[:, :, i].contiguous() for i in range(3))
    base = ra.ring_attn_func(q, k, v, layout="zigzag", world=N)
    kv = qkv[:, :, 1:]
    a = ra.ring_attn_kvpacked_func(q, kv, layout="zigzag", world=N)
    b = ra.ring_attn_qkvpacked_func(qkv, layout="zigzag", world=N)
    torch.cuda.synchronize()
    assert torch.equal(base, a) and torch.equal(base, b)
    # the block step itself on strided (packed) views, no copies
    pm = ra.posmap([(0, 1, S)])
    o1, l1 = ra.block_attn_fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], pm, pm, seq_len=S, causal=True)
    o2, l2 = ra.block_attn_fwd(q, k, v, pm, pm, seq_len=S, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt,layout", [("bf16", "contiguous"), ("f32", "contiguous"),
                                       ("bf16", "zigzag_varlen"), ("f32", "stripe_varlen")])
def test_varlen_func_autograd(dt, layout):
    import torch
    ra = _ra()
    log(f"varlen func {dt} {layout}")
    N = 4
    if layout == "contiguous":
        lengths = [7, 1, 300, 129, 1, 586]
    else:  # per-sequence layouts: lengths divisible by 2N / N
        u = 2 * N if layout == "zigzag_varlen" else N
        lengths = [u, 38 * u, 16 * u, u, 72 * u]
    T, H, D = sum(lengths), 2, 128
    cu = synth.cu_seqlens(lengths)
    q, k, v, do = synth.qkv(T, H, D, _dt(dt), seed=47, device="cpu", with_dout=True)
    q, k, v, do = (x[0].to(dev()) for x in (q, k, v, do))  # [T, h, d]
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = ra.ring_attn_varlen_func(qg, kg, vg, cu, layout=layout, world=N)
    out.backward(do)
    torch.cuda.synchronize()
    pos = np.arange(T)
    q64, k64, v64, do64 = (f64(x)[None] for x in (q, k, v, do))
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True, cu)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, True, cu)
    bf = dt == "bf16"
    check_out(f64(out)[None], ro, bf)
    check_grad(f64(qg.grad)[None], gq, bf, what="dq")
    check_grad(f64(kg.grad)[None], gk, bf, what="dk")
    check_grad(f64(vg.grad)[None], gv, bf, what="dv")


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
def test_gathered_share(layout):
    """llama3-style share: a rank's queries against all gathered K/V in one block step."""
    import torch
    ra = _ra()
    log(f"gathered share {layout}")
    S, H, D, N, r = 2048, 2, 128, 8, 3
    q, k, v = synth.qkv(S, H, D, torch.bfloat16, seed=53, device="cpu")
    q, k, v = q.to(dev()), k.to(dev()), v.to(dev())
    idx = torch.from_numpy(ra.layout_positions(layout, S, N, r)).to(dev())
    out, lse = ra.gathered_share_attn(q.index_select(1, idx).contiguous(), k, v, layout=layout, world=N, rank=r)
    torch.cuda.synchronize()
    pos = oracle.layout_positions(layout, S, N, r)
    ro, rl = oracle.attention(f64(q)[:, pos], f64(k), f64(v), pos, np.arange(S), True)
    check_out(f64(out), ro, True)
    check_lse(f64(lse), rl, True)
