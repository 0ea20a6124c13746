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


@pytest.mark.parametrize("form", ["kvpacked", "qkvpacked"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_packed_forms_gradients(form, dt):
    """Gradients flow through the packed forms' strided views into the packed
    tensor itself, and equal the oracle's gradients."""
    import torch
    ra = _ra()
    log(f"packed gradients {form} {dt}")
    S, H, D, N = 768, 2, 128, 4
    qkv, do = synth.draw_normal([(1, S, 3, H, D), (1, S, H, D)], _dt(dt), seed=45, device="cpu")
    qkv, do = qkv.to(dev()), do.to(dev())
    if form == "qkvpacked":
        x = qkv.clone().requires_grad_(True)
        out = ra.ring_attn_qkvpacked_func(x, layout="stripe", world=N)
        out.backward(do)
        grads = [x.grad[:, :, i] for i in range(3)]
    else:
        qg = qkv[:, :, 0].clone().requires_grad_(True)
        kv = qkv[:, :, 1:].clone().requires_grad_(True)
        out = ra.ring_attn_kvpacked_func(qg, kv, layout="stripe", world=N)
        out.backward(do)
        grads = [qg.grad, kv.grad[:, :, 0], kv.grad[:, :, 1]]
    torch.cuda.synchronize()
    q64, k64, v64 = (f64(qkv[:, :, i]) for i in range(3))
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, f64(do), pos, pos, True)
    bf = dt == "bf16"
    check_out(f64(out), ro, bf)
    for name, g, ref in zip(("dq", "dk", "dv"), grads, (gq, gk, gv)):
        assert g.dtype == qkv.dtype
        check_grad(f64(g), ref, bf, what=name)


@pytest.mark.parametrize("store_ds", [True, False], ids=["ds", "recompute"])
@pytest.mark.parametrize("layout,dt", [("contiguous", "bf16"), ("zigzag", "bf16"), ("stripe", "bf16"),
                                       ("zigzag", "f32")])
def test_gathered_share(layout, dt, store_ds):
    """llama3-style share: a rank's queries against all gathered K/V in one block
    step, forward and backward (this rank's contributions to dK/dV), through the
    C ABI on both dQ paths."""
    import torch
    ra = _ra()
    if dt == "f32" and not store_ds:
        pytest.skip("fp32 has one backward path")
    log(f"gathered share {layout} {dt} store_ds={store_ds}")
    S, H, D, N, r = 2048, 2, 128, 8, 3
    q, k, v, do = synth.qkv(S, H, D, _dt(dt), seed=53, device="cpu", with_dout=True)
    q, k, v, do = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    idx = torch.from_numpy(ra.layout_positions(layout, S, N, r)).to(dev())
    ql = q.index_select(1, idx).contiguous()
    dol = do.index_select(1, idx).contiguous()
    out, lse, lowp = ra.gathered_fwd(layout, N, r, ql, k, v, causal=True, want_lowp=True)
    dq, dk, dv = ra.gathered_bwd(layout, N, r, ql, k, v, out, lse, dol, causal=True, store_ds=store_ds)
    torch.cuda.synchronize()
    pos = oracle.layout_positions(layout, S, N, r)
    q64 = f64(q)[:, pos]
    ro, rl = oracle.attention(q64, f64(k), f64(v), pos, np.arange(S), True)
    gq, gk, gv = oracle.attention_backward(q64, f64(k), f64(v), ro, rl, f64(do)[:, pos], pos, np.arange(S), True)
    bf = dt == "bf16"
    check_out(f64(out), ro, bf)
    check_out(f64(lowp), ro, bf, what="out_lowp")
    check_lse(f64(lse), rl, bf)
    check_grad(f64(dq), gq, bf, what="dq")
    check_grad(f64(dk), gk, bf, what="dk")
    check_grad(f64(dv), gv, bf, what="dv")


@pytest.mark.parametrize("dt,causal", [("bf16", True), ("f32", True), ("bf16", False)])
def test_llama3_varlen_autograd(dt, causal):
    """Packed sequences through the llama3-style group (every rank's contiguous
    query slice against all gathered K/V of its sequences), with autograd, against
    full varlen attention and its gradients."""
    import torch
    ra = _ra()
    log(f"llama3 varlen {dt} causal={causal}")
    N = 4
    lengths = [7, 1, 300, 129, 1, 586, 1000]
    T, H, D = sum(lengths) + (-sum(lengths)) % N, 2, 128
    lengths[-1] += T - sum(lengths)
    cu = synth.cu_seqlens(lengths)
    q, k, v, do = synth.qkv(T, H, D, _dt(dt), seed=59, device="cpu", with_dout=True)
    q, k, v, do = (x[0].to(dev()) for x in (q, k, v, do))  # [T, h, d]
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    out, lse = ra.llama3_attn_varlen_func(qg, kg, vg, cu, world=N, causal=causal, return_lse=True)
    out.backward(do)
    torch.cuda.synchronize()
    pos = np.arange(T)
    q64, k64, v64, do64 = (f64(x)[None] for x in (q, k, v, do))
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, causal, cu)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, causal, cu)
    bf = dt == "bf16"
    check_out(f64(out)[None], ro, bf)
    check_lse(f64(lse), rl, bf)
    check_grad(f64(qg.grad)[None], gq, bf, what="dq")
    check_grad(f64(kg.grad)[None], gk, bf, what="dk")
    check_grad(f64(vg.grad)[None], gv, bf, what="dv")


@pytest.mark.parametrize("layout", ["zigzag", "stripe"])
def test_gathered_attn_func_matches_ring(layout):
    """The llama3-style group and the virtual ring compute the same attention:
    forward bit-for-bit is not expected (different key splits), parity with the
    oracle for both, and the same gradients within the bf16 bound."""
    import torch
    ra = _ra()
    log(f"gathered group vs ring {layout}")
    S, H, D, N = 1024, 2, 64, 4
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=61, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    res = []
    for fn in (ra.gathered_attn_func, ra.ring_attn_func):
        qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
        out = fn(qg, kg, vg, layout=layout, world=N, causal=True)
        out.backward(do)
        res.append((out, qg.grad, kg.grad, vg.grad))
    torch.cuda.synchronize()
    pos = np.arange(S)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), pos, pos, True)
    gq, gk, gv = oracle.attention_backward(f64(q), f64(k), f64(v), ro, rl, f64(do), pos, pos, True)
    for out, dq, dk, dv in res:
        check_out(f64(out), ro, True)
        check_grad(f64(dq), gq, True, what="dq")
        check_grad(f64(dk), gk, True, what="dk")
        check_grad(f64(dv), gv, True, what="dv")


@pytest.mark.parametrize("layout", ["contiguous", "zigzag_varlen"])
def test_cu_seqlens_holder_same_results(layout):
    """ra.CuSeqlens (host and device copies made once) gives the same bits as a
    plain cu_seqlens array in the ring forward and backward."""
    import torch
    ra = _ra()
    log(f"CuSeqlens holder {layout}")
    N = 4
    lengths = [8, 24, 200, 8, 72] if layout == "zigzag_varlen" else [7, 1, 300, 129, 1, 586]
    S, H, D = sum(lengths), 2, 128
    cu = synth.cu_seqlens(lengths)
    holder = ra.CuSeqlens(cu, dev())
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=48, device=dev(), with_dout=True)
    idx = [torch.from_numpy(ra.layout_positions(layout, S, N, r, holder)).to(dev()) for r in range(N)]
    k_ring = torch.stack([k.index_select(1, i) for i in idx]).contiguous()
    v_ring = torch.stack([v.index_select(1, i) for i in idx]).contiguous()
    r = 1
    ql, dol = q.index_select(1, idx[r]).contiguous(), do.index_select(1, idx[r]).contiguous()
    res = []
    for c in (cu, holder):
        o, l, _ = ra.ring_fwd(layout, N, r, ql, k_ring, v_ring, cu_seqlens=c)
        dq, dk, dv = ra.ring_bwd(layout, N, r, ql, k_ring, v_ring, o, l, dol, cu_seqlens=c)
        res.append((o, l, dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)
