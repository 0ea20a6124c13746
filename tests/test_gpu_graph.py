"""HIP graph capture of the virtual ring: ra_ring_fwd and ra_ring_bwd enqueue
kernels only (no allocation, no memset, no synchronisation), so a whole
forward + backward step can be captured once and replayed.  Every replay must
reproduce the eager result bit for bit (the bf16 path has no atomics), with
eager work and synchronisations between the replays."""
import pytest

import synth
from gpu_util import dev, log, ring_from_global

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout,rank", [("zigzag", 1), ("stripe", 2), ("contiguous", 3)])
def test_ring_fwd_bwd_graph_replays(layout, rank):
    import torch
    import exact_long_context_ra_amd as ra
    S, N, H, D = 4096, 4, 4, 128
    log(f"graph replay {layout} S={S} N={N} rank={rank}")
    q, k, v, do = synth.qkv(S, H, D, torch.bfloat16, seed=3, device=dev(), with_dout=True)
    kr, idx = ring_from_global(k, layout, N)
    vr, _ = ring_from_global(v, layout, N)
    ql = q.index_select(1, idx[rank]).contiguous()
    dol = do.index_select(1, idx[rank]).contiguous()
    L = S // N
    out = torch.empty((1, L, H, D), device=dev(), dtype=torch.float32)
    lse = torch.empty((1, H, L), device=dev(), dtype=torch.float32)
    lowp = torch.empty_like(ql)
    dq = torch.empty_like(out)
    dk = torch.zeros(kr.shape, device=dev(), dtype=torch.float32)
    dv = torch.zeros_like(dk)
    ws = torch.empty(ra.ring_workspace_bytes(layout, N, ql), device=dev(), dtype=torch.uint8)
    bufs = {"out": out, "lse": lse, "out_lowp": lowp, "dq": dq, "dk_ring": dk, "dv_ring": dv}

    def step():
        dk.zero_()  # a fill kernel, not a memset node
        dv.zero_()
        ra.ring_fwd(layout, N, rank, ql, kr, vr, out=out, lse=lse, out_lowp=lowp)
        ra.ring_bwd(layout, N, rank, ql, kr, vr, out, lse, dol, dq=dq, dk_ring=dk, dv_ring=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = {name: t.clone() for name, t in bufs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i in range(3):
        for t in bufs.values():
            t.fill_(float("nan"))  # eager work between replays; a replay must rewrite everything
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in bufs.items():
            assert torch.equal(t, ref[name]), f"replay {i}: {name} differs from the eager result"
    log(f"graph replay {layout}: 3 replays bit-identical to eager")
