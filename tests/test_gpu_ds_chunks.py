"""The stored-dS backward in key chunks: with a workspace that holds the dS^T of
only part of a block, the dK/dV kernel and the dQ-from-dS kernel run once per
chunk of keys.  dK/dV of a key come from its own chunk alone, so they must be
bit-identical to the one-chunk path; dQ adds the chunks one after another, so
it must agree to fp32 rounding; and both must match the float64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_grad, dev, f64, log, ring_from_global

pytestmark = pytest.mark.gpu

MIN_CHUNK = 1024  # keys: the smallest chunk the library takes


def _ra():
    import exact_long_context_ra_amd as ra
    return ra


def _per_key_bytes(B, H, L):
    return B * H * ((L + 127) // 128 * 128) * 2


# chunk sizes: a zigzag chunk that straddles the two local chunks of the layout
# (1152 keys against 2048-key halves), a strided stripe map, a plain one
@pytest.mark.parametrize("layout,S,N,chunk", [("zigzag", 8192, 2, 1152), ("stripe", 6144, 2, 1024),
                                              ("contiguous", 8192, 2, 2048)])
def test_ring_bwd_chunked(layout, S, N, chunk):
    import torch
    ra = _ra()
    H, D = 2, 128
    L = S // N
    log(f"ds chunks ring {layout} S={S} N={N} chunk={chunk}")
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=41, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    kr, idx = ring_from_global(k, layout, N)
    vr, _ = ring_from_global(v, layout, N)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    pos = np.arange(S)
    ro, rl = oracle.attention(q64, k64, v64, pos, pos, True, None)
    gq, gk, gv = oracle.attention_backward(q64, k64, v64, ro, rl, do64, pos, pos, True, None)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr)
        need = ra.ring_workspace_bytes(layout, N, ql, minimal=True)
        full = ra.ring_workspace_bytes(layout, N, ql)
        assert full == need + ((L + 127) // 128 * 128) * _per_key_bytes(1, H, L)
        # room for `chunk` keys of dS^T and a little less than one more key tile
        ws = torch.empty(need + chunk * _per_key_bytes(1, H, L) + 1000, device=dev(), dtype=torch.uint8)
        whole = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol)
        parts = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, workspace=ws)
        ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, workspace=ws, dk_ring=dk_ring, dv_ring=dv_ring)
        torch.cuda.synchronize()
        assert torch.equal(parts[1], whole[1]) and torch.equal(parts[2], whole[2]), \
            f"r={r}: dK/dV of a chunk depend on it alone"
        assert torch.allclose(parts[0], whole[0], rtol=1e-5, atol=1e-6), f"r={r}: dQ is the chunks' sum"
        check_grad(f64(parts[0]), gq[:, oracle.layout_positions(layout, S, N, r)], True, what=f"dq r={r}")
    check_grad(f64(dk_ring), oracle.to_ring(gk, layout, N), True, what="dk (all ranks, chunked)")
    check_grad(f64(dv_ring), oracle.to_ring(gv, layout, N), True, what="dv (all ranks, chunked)")


def test_gathered_bwd_chunked_matches_whole_block():
    import torch
    ra = _ra()
    S, N, H, D, rank = 8192, 2, 2, 128, 1
    L = S // N
    lengths = [300, 2500, 1, 4000, 1391]
    cu = synth.cu_seqlens(lengths)
    log(f"ds chunks gathered S={S} cu={cu.tolist()}")
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=42, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    holder = ra.CuSeqlens(cu, dev())
    idx = torch.from_numpy(ra.layout_positions("contiguous", S, N, rank)).to(dev())
    ql, dol = q.index_select(1, idx).contiguous(), do.index_select(1, idx).contiguous()
    out, lse, _ = ra.gathered_fwd("contiguous", N, rank, ql, k, v, cu_seqlens=holder)
    need = ra.gathered_workspace_bytes("contiguous", N, rank, ql, cu_seqlens=holder, minimal=True)
    ws_chunk = torch.empty(need + MIN_CHUNK * _per_key_bytes(1, H, L), device=dev(), dtype=torch.uint8)
    whole = ra.gathered_bwd("contiguous", N, rank, ql, k, v, out, lse, dol, cu_seqlens=holder)
    parts = ra.gathered_bwd("contiguous", N, rank, ql, k, v, out, lse, dol, cu_seqlens=holder, workspace=ws_chunk)
    torch.cuda.synchronize()
    assert torch.equal(parts[1], whole[1]) and torch.equal(parts[2], whole[2])
    assert torch.allclose(parts[0], whole[0], rtol=1e-5, atol=1e-6)
    pos = np.arange(S)
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    opos = idx.cpu().numpy()
    ro, rl = oracle.attention(q64[:, opos], k64, v64, opos, pos, True, cu)
    gq, gk, gv = oracle.attention_backward(q64[:, opos], k64, v64, ro, rl, do64[:, opos], opos, pos, True, cu)
    check_grad(f64(parts[0]), gq, True, what="dq (chunked)")
    check_grad(f64(parts[1]), gk, True, what="dk (chunked)")
    check_grad(f64(parts[2]), gv, True, what="dv (chunked)")
