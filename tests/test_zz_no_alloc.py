"""ra_ring_bwd_noalloc (the backward for callers that cannot allocate: its
scratch is a fixed per-GPU device array) against ra_ring_bwd with a caller
workspace: same kernels, so the same bits.  Two calls in a row, the second
with a smaller problem, and both dQ paths (stored dS^T when it fits the
scratch, the recompute kernel when only delta fits)."""
import numpy as np
import pytest

import synth
from gpu_util import dev, log, ring_from_global

pytestmark = pytest.mark.gpu


def _run_pair(ra, layout, S, N, H, D, dtype, rank, cu=None, seed=3):
    import torch
    q, k, v, do = synth.qkv(S, H, D, dtype, seed=seed, device="cpu", with_dout=True)
    q, k, v, do = (x.to(dev()) for x in (q, k, v, do))
    kr, idx = ring_from_global(k, layout, N, cu)
    vr, _ = ring_from_global(v, layout, N, cu)
    ql = q.index_select(1, idx[rank]).contiguous()
    dol = do.index_select(1, idx[rank]).contiguous()
    out, lse, _ = ra.ring_fwd(layout, N, rank, ql, kr, vr, causal=True, cu_seqlens=cu)
    L = S // N
    # the path the scratch allows: stored dS^T when delta and dS^T both fit, else recompute
    need_full = ra.ring_workspace_bytes(layout, N, ql, cu_seqlens=cu)
    store_ds = need_full <= ra.noalloc_scratch_bytes()
    ref = ra.ring_bwd(layout, N, rank, ql, kr, vr, out, lse, dol, causal=True, cu_seqlens=cu, store_ds=store_ds)
    dq = torch.full((1, L, H, D), float("nan"), device=dev(), dtype=torch.float32)
    dk = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv = torch.zeros(vr.shape, device=dev(), dtype=torch.float32)
    got = ra.ring_bwd_noalloc(layout, N, rank, ql, kr, vr, out, lse, dol, dq, dk, dv, causal=True,
                              cu_seqlens=None if cu is None else np.asarray(cu))
    torch.cuda.synchronize()
    return ref, got, store_ds


@pytest.mark.parametrize("layout", ["zigzag", "stripe"])
def test_noalloc_matches_workspace_path(layout):
    import torch
    import exact_long_context_ra_amd as ra
    # (S, N, H): dS^T fits the scratch; then smaller; then only delta fits; then smaller again
    for S, N, H in ((2048, 4, 2), (1024, 4, 2), (32768, 8, 32), (16384, 8, 32)):
        ref, got, store_ds = _run_pair(ra, layout, S, N, H, 128, torch.bfloat16, rank=1)
        log(f"noalloc {layout} S={S} N={N} H={H} stored dS^T={store_ds}")
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs from ra_ring_bwd ({layout} S={S} H={H})"


def test_noalloc_per_sequence_fp32():
    """fp32 per-sequence layout: the no-allocation call runs the sequences one after
    another on the caller's stream (ra_ring_bwd uses side streams); fp32 dQ is
    accumulated with atomics, so it matches to rounding, dK/dV exactly."""
    import torch
    import exact_long_context_ra_amd as ra
    from gpu_util import varlen_cu_multiple
    for S in (1536, 768):
        N = 4
        cu = varlen_cu_multiple(S, N) if S == 1536 else synth.cu_seqlens([4, 380, 4, 380])
        log(f"noalloc stripe_varlen fp32 S={S}")
        ref, got, _ = _run_pair(ra, "stripe_varlen", S, N, 2, 64, torch.float32, rank=2, cu=cu)
        assert torch.allclose(got[0], ref[0], rtol=1e-5, atol=1e-6), "dq"
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), "dk/dv"


def test_noalloc_rejects_oversized_problem():
    import torch
    import exact_long_context_ra_amd as ra
    from exact_long_context_ra_amd import RAError
    # delta of 64 heads x 131200 rows x 4 B, more than the 32 MiB scratch.  Every
    # tensor aliases one small buffer (stride 0), so that even a call that was not
    # refused would stay inside its buffers.
    S, N, H, D = 8 * (131072 + 128), 8, 64, 128
    L = S // N

    def alias(shape, dtype):
        return torch.zeros(D, device=dev(), dtype=dtype).as_strided(shape, (0,) * (len(shape) - 1) + (1,))

    q = alias((1, L, H, D), torch.bfloat16)
    ring = alias((N, 1, L, H, D), torch.bfloat16)
    out32 = alias((1, L, H, D), torch.float32)
    grad_ring = alias((N, 1, L, H, D), torch.float32)
    lse = torch.zeros(H * L, device=dev(), dtype=torch.float32)
    with pytest.raises(RAError, match="fixed scratch"):
        ra.ring_bwd_noalloc("zigzag", N, 0, q, ring, ring, out32, lse, q, out32, grad_ring, grad_ring)
    torch.cuda.synchronize()
