"""Backward parity: HIP block/ring backward against the float64 oracle's
textbook gradients on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import varlen_cu_many, varlen_cu_multiple, check_grad, dev, f64, log, ring_from_global

pytestmark = pytest.mark.gpu


def _ra():
    import exact_long_context_ra_amd as ra
    return ra


def _dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


BLOCK_BWD_CASES = [
    # (name, lq, lk, q segments, k segments, seq_len, causal, cu)
    ("self_causal", [(0, 1, 256)], [(0, 1, 256)], 256, True, None),
    ("ragged_past", [(200, 1, 130)], [(0, 1, 190)], 330, True, None),
    ("noncausal", [(0, 1, 100)], [(0, 1, 300)], 300, False, None),
    ("zigzag_two_seg", [(64, 1, 64), (448, 1, 64)], [(0, 1, 64), (512, 1, 64)], 576, True, None),
    ("stripe_strict", [(1, 4, 150)], [(3, 4, 150)], 600, True, None),
    ("varlen", [(0, 1, 300)], [(0, 1, 300)], 300, True, [0, 1, 70, 71, 200, 300]),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", BLOCK_BWD_CASES, ids=[c[0] for c in BLOCK_BWD_CASES])
def test_block_bwd(case, D, dt):
    """A block step of the backward with the block's own final (out, lse): the
    GPU forward feeds the GPU backward; the oracle recomputes everything."""
    import torch
    ra = _ra()
    name, qsegs, ksegs, S, causal, cu = case
    log(f"block_bwd {name} D={D} {dt}")
    qpos = np.concatenate([b + s * np.arange(n) for b, s, n in qsegs])
    kpos = np.concatenate([b + s * np.arange(n) for b, s, n in ksegs])
    H, B = 2, (2 if cu is None else 1)
    lq, lk = len(qpos), len(kpos)
    q, k, v, do = synth.draw_normal([(B, lq, H, D), (B, lk, H, D), (B, lk, H, D), (B, lq, H, D)],
                                    _dtype(dt), seed=21, device="cpu")
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    qm, km = ra.posmap(qsegs), ra.posmap(ksegs)
    out, lse = ra.block_attn_fwd(q, k, v, qm, km, seq_len=S, causal=causal, cu_seqlens=cu)
    delta = ra.bwd_preprocess(out, do)
    dq = torch.zeros((B, lq, H, D), device=dev(), dtype=torch.float32)
    dk = torch.zeros((B, lk, H, D), device=dev(), dtype=torch.float32)
    dv = torch.zeros((B, lk, H, D), device=dev(), dtype=torch.float32)
    ra.block_attn_bwd(q, k, v, do, lse, delta, qm, km, dq, dk, dv, seq_len=S, causal=causal, cu_seqlens=cu)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    ro, rl = oracle.attention(q64, k64, v64, qpos, kpos, causal, cu)
    # delta against its definition with the oracle's output
    ref_delta = np.einsum("blhd,blhd->bhl", do64, ro)
    bf = dt == "bf16"
    check_grad(f64(delta), ref_delta, bf, what="delta")
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, qpos, kpos, causal, cu)
    check_grad(f64(dq), gq, bf, what="dq")
    check_grad(f64(dk), gk, bf, what="dk")
    check_grad(f64(dv), gv, bf, what="dv")


RING_BWD_CASES = [
    # (layout, S, N, H, D, dtype, cu)
    ("contiguous", 1024, 4, 2, 128, "f32", None),
    ("zigzag", 1024, 4, 2, 128, "f32", None),
    ("stripe", 1024, 4, 2, 64, "f32", None),
    ("contiguous", 1024, 4, 2, 128, "bf16", None),
    ("zigzag", 2048, 4, 2, 128, "bf16", None),
    ("stripe", 2048, 8, 2, 128, "bf16", None),
    ("zigzag", 800, 4, 2, 64, "bf16", None),
    ("contiguous", 1536, 4, 2, 128, "bf16", "varlen"),
    ("stripe", 1536, 4, 2, 128, "f32", "varlen"),
    ("zigzag", 1536, 4, 2, 128, "bf16", "varlen"),   # two-segment posmaps with sequence boundaries
    ("stripe", 1536, 8, 2, 64, "bf16", "varlen"),    # strided posmaps with sequence boundaries
    ("zigzag_varlen", 1536, 4, 2, 128, "bf16", "varlen"),
    ("stripe_varlen", 1536, 4, 2, 64, "bf16", "varlen"),
    ("zigzag_varlen", 1536, 4, 2, 64, "f32", "varlen"),
    ("zigzag_varlen", 2048, 4, 2, 128, "bf16", "many"),   # 21 sequences: two grouped launches per step
]


# bf16 runs both dQ paths: from the dS the dK/dV kernel stores (full workspace)
# and by recomputing S and dP (minimal workspace); fp32 has one path.
RING_BWD_RUNS = [(c, True) for c in RING_BWD_CASES] + [(c, False) for c in RING_BWD_CASES if c[5] == "bf16"]


@pytest.mark.parametrize("case,store_ds", RING_BWD_RUNS,
                         ids=lambda c: "-".join(str(x) for x in c) if isinstance(c, tuple) else
                         ("ds" if c else "recompute"))
def test_ring_bwd(case, store_ds):
    """Every rank runs fwd then bwd into shared dK/dV ring buffers: per-rank dQ
    and the summed dK/dV must equal the full-sequence gradients."""
    import torch
    ra = _ra()
    layout, S, N, H, D, dt, cu = case
    log(f"ring_bwd {case} store_ds={store_ds}")
    if cu == "many":
        cu = varlen_cu_many(S, 2 * N if layout == "zigzag_varlen" else N)
    elif cu == "varlen" and layout.endswith("_varlen"):
        cu = varlen_cu_multiple(S, 2 * N if layout == "zigzag_varlen" else N)
    elif cu == "varlen":
        lengths = [1, 200, 1, 129, 300]
        lengths.append(S - sum(lengths))
        cu = synth.cu_seqlens(lengths)
    q, k, v, do = synth.qkv(S, H, D, _dtype(dt), seed=31, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    kr, idx = ring_from_global(k, layout, N, cu)
    vr, _ = ring_from_global(v, layout, N, cu)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True, cu)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, True, cu)
    bf = dt == "bf16"
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, cu_seqlens=cu)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=True, cu_seqlens=cu,
                               dk_ring=dk_ring, dv_ring=dv_ring, store_ds=store_ds)
        torch.cuda.synchronize()
        opos = oracle.layout_positions(layout, S, N, r, cu)
        check_grad(f64(dq), gq[:, opos], bf, what=f"dq r={r}")
    check_grad(f64(dk_ring), oracle.to_ring(gk, layout, N, cu), bf, what="dk (all ranks)")
    check_grad(f64(dv_ring), oracle.to_ring(gv, layout, N, cu), bf, what="dv (all ranks)")


@pytest.mark.parametrize("store_ds", [True, False], ids=["ds", "recompute"])
@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
def test_ring_bwd_noncausal(layout, store_ds):
    """Without the causal mask every ring step is a fully visible block (the
    layouts then only permute tokens): per-rank dQ and the summed dK/dV must
    equal the gradients of full attention."""
    import torch
    ra = _ra()
    S, N, H, D = 1024, 4, 2, 128
    log(f"ring_bwd noncausal {layout} store_ds={store_ds}")
    q, k, v, do = synth.qkv(S, H, D, _dtype("bf16"), seed=33, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    kr, idx = ring_from_global(k, layout, N, None)
    vr, _ = ring_from_global(v, layout, N, None)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, False)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, False)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=False)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=False,
                               dk_ring=dk_ring, dv_ring=dv_ring, store_ds=store_ds)
        torch.cuda.synchronize()
        opos = oracle.layout_positions(layout, S, N, r)
        check_grad(f64(dq), gq[:, opos], True, what=f"dq r={r}")
    check_grad(f64(dk_ring), oracle.to_ring(gk, layout, N), True, what="dk (all ranks)")
    check_grad(f64(dv_ring), oracle.to_ring(gv, layout, N), True, what="dv (all ranks)")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ring_per_sequence_on_user_stream(dt):
    """The per-sequence layouts run every sequence as a ring of its own: bf16
    in grouped launches (one per step over all sequences), fp32 on side
    streams forked from and joined back into the caller's stream.  Called on a
    user stream, with the results consumed on that stream before any
    device-wide synchronisation, forward and backward (both dQ paths) give
    bit-identical results to a default-stream run."""
    import torch
    ra = _ra()
    layout, S, N, H, D = "zigzag_varlen", 2048, 4, 2, 128
    log(f"ring per-sequence on a user stream {layout} S={S} {dt}")
    cu = varlen_cu_multiple(S, 2 * N)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v, do = synth.qkv(S, H, D, dtype, seed=7, device="cpu", with_dout=True)
    q, k, v, do = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    kr, idx = ring_from_global(k, layout, N, cu)
    vr, _ = ring_from_global(v, layout, N, cu)
    r = 1
    ql = q.index_select(1, idx[r]).contiguous()
    dol = do.index_select(1, idx[r]).contiguous()

    def run(store_ds):
        o, l, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, cu_seqlens=cu)
        dq, dk, dv = ra.ring_bwd(layout, N, r, ql, kr, vr, o, l, dol, causal=True, cu_seqlens=cu,
                                 store_ds=store_ds)
        sums = torch.stack([t.double().sum() for t in (o, l.clamp(min=-1e30), dq, dk, dv)])
        return (o, l, dq, dk, dv), sums

    for store_ds in ((True, False) if dt == "bf16" else (True,)):
        ref, _ = run(store_ds)
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            got, sums = run(store_ds)
        st.synchronize()
        # fp32 dQ is accumulated with float atomics (order-dependent rounding)
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), got, ref):
            if dt == "f32" and name == "dq":
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-6), f"dq differs on a user stream ({dt})"
            else:
                assert torch.equal(a, b), f"{name} differs on a user stream (store_ds={store_ds})"
        ref_sums = torch.stack([t.double().sum() for t in (ref[0], ref[1].clamp(min=-1e30), *ref[2:])])
        assert torch.allclose(sums, ref_sums, rtol=1e-9 if dt == "bf16" else 1e-6, atol=0), \
            "results consumed on the user stream before the join completed"
        torch.cuda.synchronize()


@pytest.mark.parametrize("store_ds", [True, False], ids=["ds", "recompute"])
@pytest.mark.parametrize("dt,layout", [("bf16", "zigzag"), ("bf16", "stripe"), ("f32", "zigzag"),
                                       ("f32", "contiguous")])
def test_ring_softmax_scale(dt, layout, store_ds):
    """An explicit softmax_scale through the ring forward and backward (every rank,
    summed dK/dV) against the oracle with the same scale."""
    import torch
    ra = _ra()
    if dt == "f32" and not store_ds:
        pytest.skip("fp32 has one backward path")
    scale, S, N, H, D = 0.05, 1024, 4, 2, 128
    log(f"ring scale={scale} {layout} {dt} store_ds={store_ds}")
    q, k, v, do = synth.qkv(S, H, D, _dtype(dt), seed=37, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    kr, idx = ring_from_global(k, layout, N)
    vr, _ = ring_from_global(v, layout, N)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True, scale=scale)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, True, scale=scale)
    bf = dt == "bf16"
    from gpu_util import check_lse, check_out
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, scale=scale)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=True, scale=scale,
                               dk_ring=dk_ring, dv_ring=dv_ring, store_ds=store_ds)
        torch.cuda.synchronize()
        opos = oracle.layout_positions(layout, S, N, r)
        check_out(f64(out), ro[:, opos], bf, what=f"out r={r}")
        check_lse(f64(lse), rl[:, :, opos], bf, what=f"lse r={r}")
        check_grad(f64(dq), gq[:, opos], bf, what=f"dq r={r}")
    check_grad(f64(dk_ring), oracle.to_ring(gk, layout, N), bf, what="dk (all ranks)")
    check_grad(f64(dv_ring), oracle.to_ring(gv, layout, N), bf, what="dv (all ranks)")
