"""Parity at the full benchmark sizes (32 heads, head_dim 128, bf16 N(0,1)),
in the launch configuration the benchmark times (ra_ring_fwd / ra_ring_bwd on
resident rank-major K/V rings).

The float64 oracle cannot redo every output at these sizes, so:
* forward: sampled query rows (tile, chunk and segment boundaries plus seeded
  random rows) on sampled heads are recomputed exactly by the oracle;
* backward: dQ of sampled rows is recomputed exactly (a row's dQ depends only
  on that row), and dK/dV are checked on every head through identities that
  hold at any size: the rank's contributions satisfy sum_j dK_j = 0 and
  sum_j dV_j = sum_i dO_i (each row of P sums to one, each row of dS to zero).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_grad, check_lse, check_out, dev, f64, log, oracle_rows_fwd_bwd, ring_from_global

pytestmark = pytest.mark.gpu

H, D = 32, 128
HEADS = [0, 17, 31]
TAIL_REL = 3e-2


def _ra():
    import exact_long_context_ra_amd as ra
    return ra


def _sample_rows(L, seed, extra=()):
    base = {0, 1, 31, 32, 63, 64, 127, 128, L // 2 - 1, L // 2, L - 2, L - 1, *extra}
    rng = np.random.default_rng(seed)
    base.update(rng.integers(0, L, 16).tolist())
    return np.array(sorted(r for r in base if 0 <= r < L), dtype=np.int64)


def _setup(layout, S, N, seed, cu=None):
    import torch
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=seed, device=dev(), with_dout=True)
    kr, idx = ring_from_global(k, layout, N, cu)
    vr, _ = ring_from_global(v, layout, N, cu)
    # host float64 copies of the sampled heads only
    hsel = torch.tensor(HEADS, device=dev())
    k64 = f64(k.index_select(2, hsel))
    v64 = f64(v.index_select(2, hsel))
    return q, do, kr, vr, idx, k64, v64, hsel


def _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, cu, what):
    import torch
    S = k64.shape[1]
    gidx = torch.from_numpy(pos[rows]).to(q.device)
    qr = f64(q.index_select(2, hsel).index_select(1, gidx))
    ro, rl = oracle.attention(qr, k64, v64, pos[rows], np.arange(S), True, cu)
    got_o = f64(out.index_select(2, hsel))[:, rows]
    got_l = f64(lse.index_select(1, hsel))[:, :, rows]
    check_out(got_o, ro, True, what=f"{what} out")
    check_lse(got_l, rl, True, what=f"{what} lse")
    return ro, rl


def _check_invariants(dk_ring, dv_ring, dol, out_has_keys, what):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i over the rank's rows (per head, per d)."""
    dk = dk_ring.double().sum(dim=(0, 2))   # [b, h, d]
    dv = dv_ring.double().sum(dim=(0, 2))
    dks = dk_ring.double().abs().sum(dim=(0, 2))
    dvs = dv_ring.double().abs().sum(dim=(0, 2))
    want_dv = (dol.double() * out_has_keys[None, :, None, None]).sum(dim=1)
    err_k = float((dk.abs() / (dks + 1e-30)).max())
    err_v = float(((dv - want_dv).abs() / (dvs + 1e-30)).max())
    log(f"{what}: sum dK rel {err_k:.2e}, sum dV rel {err_v:.2e}")
    assert err_k <= 1e-3, f"{what}: sum_j dK_j = {err_k:.3e} of sum |dK|"
    assert err_v <= 1e-3, f"{what}: sum_j dV_j - sum_i dO_i = {err_v:.3e} of sum |dV|"


def _check_dq_rows(q, do, dq, out_rows_ref, lse_rows_ref, pos, rows, k64, v64, hsel, cu, what):
    import torch
    S = k64.shape[1]
    gidx = torch.from_numpy(pos[rows]).to(q.device)
    qr = f64(q.index_select(2, hsel).index_select(1, gidx))
    dor = f64(do.index_select(2, hsel).index_select(1, gidx))
    gq, _, _ = oracle.attention_backward(qr, k64, v64, out_rows_ref, lse_rows_ref, dor, pos[rows], np.arange(S),
                                         True, cu)
    check_grad(f64(dq.index_select(2, hsel))[:, rows], gq, True, what=f"{what} dq")


def _check_tail_dkdv(q, do, dk_ring, dv_ring, pos, idx, k64, v64, hsel, what, tail=96):
    """Exact dK/dV for the keys that only the share's last `tail` query rows
    (by position) see: under the causal mask a key at position p is seen by the
    rows at positions >= p, so for every key past the position of the
    (tail+1)-th last row all of its viewers are among those rows, and the
    oracle needs the forward of those rows alone.  dk_ring/dv_ring hold this
    rank's contributions only."""
    import torch
    S = k64.shape[1]
    order = np.argsort(pos)
    rows = np.sort(order[-tail:])
    thr = int(pos[order[-tail - 1]])
    kpos = np.arange(thr + 1, int(pos.max()) + 1)
    gidx = torch.from_numpy(pos[rows]).to(q.device)
    qr = f64(q.index_select(2, hsel).index_select(1, gidx))
    dor = f64(do.index_select(2, hsel).index_select(1, gidx))
    ro, rl = oracle.attention(qr, k64, v64, pos[rows], np.arange(S), True)
    _, gk, gv = oracle.attention_backward(qr, k64[:, kpos], v64[:, kpos], ro, rl, dor, pos[rows], kpos, True)
    # global position -> row of the rank-major ring
    inv = np.empty(S, dtype=np.int64)
    inv[torch.cat(idx).cpu().numpy()] = np.arange(S)
    ring_rows = torch.from_numpy(inv[kpos]).to(q.device)
    N, B, L = dk_ring.shape[:3]
    got_k = f64(dk_ring.reshape(N * L, *dk_ring.shape[3:]).index_select(0, ring_rows).index_select(1, hsel))[None]
    got_v = f64(dv_ring.reshape(N * L, *dv_ring.shape[3:]).index_select(0, ring_rows).index_select(1, hsel))[None]
    # These gradients are sums over a few rows, far below 1 in magnitude, so the
    # bound is relative to their own largest value: bf16 P and dS carry 2^-9
    # relative rounding per term, and TAIL_REL leaves room for cancellation.
    for name, got, ref in (("dk", got_k, gk), ("dv", got_v, gv)):
        mx = float(np.max(np.abs(ref)))
        rel = float(np.max(np.abs(got - ref))) / mx
        log(f"{what}: {name} of {len(kpos)} keys seen only by the last {tail} rows: max err {rel:.2e} of max|ref|")
        assert rel <= TAIL_REL, f"{what} {name} tail: max abs err {rel:.3e} of max|ref| {mx:.3e} > {TAIL_REL}"


@pytest.mark.parametrize("layout,S,rank", [("zigzag", 131072, 0), ("zigzag", 131072, 5),
                                           ("stripe", 262144, 0),
                                           # one million tokens: the backward's dS^T in 32 key chunks per step
                                           ("zigzag", 1048576, 0)])
def test_full_size_fwd_bwd(layout, S, rank):
    import torch
    ra = _ra()
    N = 8
    log(f"full-size {layout} S={S} rank={rank}")
    q, do, kr, vr, idx, k64, v64, hsel = _setup(layout, S, N, seed=0)
    ql = q.index_select(1, idx[rank]).contiguous()
    dol = do.index_select(1, idx[rank]).contiguous()
    out, lse, _ = ra.ring_fwd(layout, N, rank, ql, kr, vr, causal=True)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    dq, _, _ = ra.ring_bwd(layout, N, rank, ql, kr, vr, out, lse, dol, causal=True, dk_ring=dk_ring,
                           dv_ring=dv_ring)
    torch.cuda.synchronize()
    pos = oracle.layout_positions(layout, S, N, rank)
    L = S // N
    rows = _sample_rows(L, seed=rank + 1, extra=(L // 2 + 1,))
    # q/do are the global tensors: the checks take rows by global position
    ro, rl = _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, None, f"{layout} r{rank}")
    _check_dq_rows(q, do, dq, ro, rl, pos, rows, k64, v64, hsel, None, f"{layout} r{rank}")
    has = torch.ones(L, device=dev(), dtype=torch.float64)  # causal self-attention: every row sees itself
    _check_invariants(dk_ring, dv_ring, dol, has, f"{layout} r{rank}")
    _check_tail_dkdv(q, do, dk_ring, dv_ring, pos, idx, k64, v64, hsel, f"{layout} r{rank}")


@pytest.mark.parametrize("layout,S,rank,heads", [("zigzag", 131072, 0, (0, 31)), ("stripe", 262144, 0, (0,))])
def test_full_size_full_heads(layout, S, rank, heads):
    """Element by element over WHOLE heads of the benchmark share: out, lse and dQ
    of every query row, and this rank's dK/dV contributions to every key of all
    N blocks, against the oracle (run on row blocks in threads), plus the sum
    identities on every head."""
    import time

    import torch
    ra = _ra()
    N = 8
    log(f"full-size full heads {layout} S={S} rank={rank} heads={heads}")
    q, do, kr, vr, idx, k64, v64, hsel = _setup(layout, S, N, seed=0)
    ql = q.index_select(1, idx[rank]).contiguous()
    dol = do.index_select(1, idx[rank]).contiguous()
    out, lse, _ = ra.ring_fwd(layout, N, rank, ql, kr, vr, causal=True)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    dq, _, _ = ra.ring_bwd(layout, N, rank, ql, kr, vr, out, lse, dol, causal=True, dk_ring=dk_ring,
                           dv_ring=dv_ring)
    torch.cuda.synchronize()
    L = S // N
    _check_invariants(dk_ring, dv_ring, dol, torch.ones(L, device=dev(), dtype=torch.float64),
                      f"{layout} r{rank}")
    pos = oracle.layout_positions(layout, S, N, rank)
    # rank-major ring rows -> global order (library positions, checked equal to the oracle's elsewhere)
    perm = torch.cat(idx)
    for h in heads:
        j = HEADS.index(h)
        t0 = time.perf_counter()
        q64 = f64(ql[:, :, h:h + 1])
        do64 = f64(dol[:, :, h:h + 1])
        ro, rl, gq, gk, gv = oracle_rows_fwd_bwd(q64, k64[:, :, j:j + 1], v64[:, :, j:j + 1], do64, pos,
                                                 np.arange(S), True)
        log(f"{layout} r{rank} head {h}: oracle {time.perf_counter() - t0:.1f} s")
        what = f"{layout} r{rank} head {h}"
        check_out(f64(out[:, :, h:h + 1]), ro, True, what=f"{what} out")
        check_lse(f64(lse[:, h:h + 1]), rl, True, what=f"{what} lse")
        check_grad(f64(dq[:, :, h:h + 1]), gq, True, what=f"{what} dq")
        dk_g = torch.empty((1, S, 1, D), device=dev(), dtype=torch.float32)
        dv_g = torch.empty((1, S, 1, D), device=dev(), dtype=torch.float32)
        dk_g[:, perm] = dk_ring[:, :, :, h:h + 1].permute(1, 0, 2, 3, 4).reshape(1, S, 1, D)
        dv_g[:, perm] = dv_ring[:, :, :, h:h + 1].permute(1, 0, 2, 3, 4).reshape(1, S, 1, D)
        ek = check_grad(f64(dk_g), gk, True, what=f"{what} dk")
        ev = check_grad(f64(dv_g), gv, True, what=f"{what} dv")
        log(f"{what}: dk max err {ek:.2e} (max|ref| {np.abs(gk).max():.2e}), dv {ev:.2e} "
            f"(max|ref| {np.abs(gv).max():.2e})")


def test_full_size_contiguous_all_ranks():
    """Contiguous causal ring over 32768 tokens: every rank's share, forward and
    backward (ranks 0 to 7 run 1 to 8 ring steps)."""
    import torch
    ra = _ra()
    layout, S, N = "contiguous", 32768, 8
    log("full-size contiguous S=32768 all ranks")
    q, do, kr, vr, idx, k64, v64, hsel = _setup(layout, S, N, seed=0)
    L = S // N
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, lowp = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, want_lowp=True)
        dk_r = torch.zeros_like(dk_ring)
        dv_r = torch.zeros_like(dv_ring)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=True, dk_ring=dk_r, dv_ring=dv_r)
        torch.cuda.synchronize()
        pos = oracle.layout_positions(layout, S, N, r)
        rows = _sample_rows(L, seed=10 + r)
        ro, rl = _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, None, f"contiguous r{r}")
        check_out(f64(lowp.index_select(2, hsel))[:, rows], ro, True, what=f"contiguous r{r} out_lowp")
        if r in (0, N - 1):
            _check_dq_rows(q, do, dq, ro, rl, pos, rows, k64, v64, hsel, None, f"contiguous r{r}")
        _check_invariants(dk_r, dv_r, dol, torch.ones(L, device=dev(), dtype=torch.float64), f"contiguous r{r}")
        dk_ring += dk_r
        dv_ring += dv_r
    _check_invariants(dk_ring, dv_ring, do.index_select(1, torch.cat(idx)), torch.ones(S, device=dev(),
                      dtype=torch.float64), "contiguous all ranks")


def test_full_size_varlen_all_slices():
    """Packed varlen (131072 tokens, log-uniform lengths in [1024, 32768], seed 0),
    8 contiguous query slices each attending to all K/V of their sequences."""
    import torch
    ra = _ra()
    layout, S, N = "contiguous", 131072, 8
    lengths = synth.loguniform_lengths(S, 1024, 32768, seed=0)
    cu = synth.cu_seqlens(lengths)
    log(f"full-size varlen {len(lengths)} sequences")
    q, do, kr, vr, idx, k64, v64, hsel = _setup(layout, S, N, seed=0, cu=cu)
    L = S // N
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, cu_seqlens=cu)
        dk_r = torch.zeros_like(dk_ring)
        dv_r = torch.zeros_like(dv_ring)
        dq, _, _ = ra.ring_bwd(layout, N, r, ql, kr, vr, out, lse, dol, causal=True, cu_seqlens=cu,
                               dk_ring=dk_r, dv_ring=dv_r)
        torch.cuda.synchronize()
        pos = oracle.layout_positions(layout, S, N, r)
        starts = [int(c) - r * L for c in cu[:-1] if r * L <= c < (r + 1) * L]
        rows = _sample_rows(L, seed=20 + r, extra=tuple(starts) + tuple(s + 1 for s in starts))
        ro, rl = _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, cu, f"varlen r{r}")
        if r in (0, 5):
            _check_dq_rows(q, do, dq, ro, rl, pos, rows, k64, v64, hsel, cu, f"varlen r{r}")
        has = torch.ones(L, device=dev(), dtype=torch.float64)
        _check_invariants(dk_r, dv_r, dol, has, f"varlen r{r}")
        dk_ring += dk_r
        dv_ring += dv_r
    # all slices together: the complete gradients, still satisfying the identities
    _check_invariants(dk_ring, dv_ring, do.index_select(1, torch.cat(idx)), torch.ones(S, device=dev(),
                      dtype=torch.float64), "varlen all slices")


@pytest.mark.parametrize("layout", ["zigzag_varlen", "stripe_varlen"])
def test_full_size_per_sequence(layout):
    """The benchmark's per-sequence share: the 13 packed sequences of the varlen
    workload (131072 tokens), every sequence a ring of 8 of its own, rank 0.
    Sampled rows include, for every sequence, its first and last local rows, the
    boundary between its two zigzag chunks and the row from which the forward
    and dQ launches start after step 0 (a multiple of 16 at or below the second
    chunk); out, lse and dQ against the oracle, dK/dV through the identities."""
    import torch
    ra = _ra()
    S, N, rank = 131072, 8, 0
    unit = 2 * N if layout == "zigzag_varlen" else N
    lengths = synth.round_lengths(synth.loguniform_lengths(S, 1024, 32768, seed=0), unit)
    cu = synth.cu_seqlens(lengths)
    log(f"full-size {layout} {len(lengths)} sequences rank {rank}")
    q, do, kr, vr, idx, k64, v64, hsel = _setup(layout, S, N, seed=0, cu=cu)
    ql = q.index_select(1, idx[rank]).contiguous()
    dol = do.index_select(1, idx[rank]).contiguous()
    out, lse, _ = ra.ring_fwd(layout, N, rank, ql, kr, vr, causal=True, cu_seqlens=cu)
    dk_ring = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv_ring = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    dq, _, _ = ra.ring_bwd(layout, N, rank, ql, kr, vr, out, lse, dol, causal=True, cu_seqlens=cu,
                           dk_ring=dk_ring, dv_ring=dv_ring)
    torch.cuda.synchronize()
    pos = oracle.layout_positions(layout, S, N, rank, cu)
    assert np.array_equal(pos, idx[rank].cpu().numpy())
    L = S // N
    extra, off = [], 0
    for n in lengths:
        loc = n // N                       # this rank's rows of the sequence
        half = loc // 2                    # zigzag: its first chunk
        extra += [off, off + 1, off + loc - 1, off + half - 1, off + half, off + half + 1, off + half // 16 * 16]
        off += loc
    rows = _sample_rows(L, seed=3, extra=tuple(extra))
    ro, rl = _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, cu, f"{layout} r{rank}")
    _check_dq_rows(q, do, dq, ro, rl, pos, rows, k64, v64, hsel, cu, f"{layout} r{rank}")
    _check_invariants(dk_ring, dv_ring, dol, torch.ones(L, device=dev(), dtype=torch.float64),
                      f"{layout} r{rank}")


def test_full_size_varlen_gathered():
    """The same packed varlen stream through the gathered-K/V share, as the
    benchmark runs it: every rank's slice against the whole K/V in one block
    step (the visible key range only), sampled rows of out, lse and dQ against
    the oracle, and dK/dV summed over all slices through the identities."""
    import torch
    ra = _ra()
    layout, S, N = "contiguous", 131072, 8
    lengths = synth.loguniform_lengths(S, 1024, 32768, seed=0)
    cu = synth.cu_seqlens(lengths)
    log(f"full-size varlen gathered {len(lengths)} sequences")
    q, do, _, _, idx, k64, v64, hsel = _setup(layout, S, N, seed=0, cu=cu)
    k, v = synth.qkv(S, H, D, torch.bfloat16, seed=0, device=dev())[1:3]
    L = S // N
    dk_all = torch.zeros((1, S, H, D), device=dev(), dtype=torch.float32)
    dv_all = torch.zeros_like(dk_all)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        dol = do.index_select(1, idx[r]).contiguous()
        out, lse, _ = ra.gathered_fwd(layout, N, r, ql, k, v, causal=True, cu_seqlens=cu)
        dq, _, _ = ra.gathered_bwd(layout, N, r, ql, k, v, out, lse, dol, causal=True, cu_seqlens=cu,
                                   dk_all=dk_all, dv_all=dv_all)
        torch.cuda.synchronize()
        pos = oracle.layout_positions(layout, S, N, r)
        starts = [int(c) - r * L for c in cu[:-1] if r * L <= c < (r + 1) * L]
        rows = _sample_rows(L, seed=30 + r, extra=tuple(starts) + tuple(s + 1 for s in starts))
        ro, rl = _check_fwd_rows(q, out, lse, pos, rows, k64, v64, hsel, cu, f"gathered r{r}")
        if r in (0, 5):
            _check_dq_rows(q, do, dq, ro, rl, pos, rows, k64, v64, hsel, cu, f"gathered r{r}")
    _check_invariants(dk_all[None], dv_all[None], do, torch.ones(S, device=dev(), dtype=torch.float64),
                      "gathered all slices")
