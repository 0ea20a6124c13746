"""The benchmark's FLOP accounting: the visible (query, key) pairs it credits
per ring step, counted with sorted searches over library positions, must equal
the pairs the oracle counts from the mask itself, for every layout, with and
without packed sequences.  The metric credits exactly these pairs (4 * d * h
FLOP each in the forward), so a miscount would misstate every bench line."""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def bench_mod():
    import bench
    return bench


@pytest.fixture(scope="module")
def ra():
    import exact_long_context_ra_amd as pkg
    pkg.lib()
    return pkg


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
@pytest.mark.parametrize("varlen", [False, True])
def test_step_pairs_match_oracle_mask(bench_mod, ra, layout, varlen):
    S, N = 512, 4
    cu = synth.cu_seqlens(synth.loguniform_lengths(S, 16, 160, seed=3)) if varlen else None
    for r in range(N):
        got = bench_mod.step_pairs(ra, layout, S, N, r, cu)
        qpos = oracle.layout_positions(layout, S, N, r)
        want = [oracle.count_pairs(qpos, oracle.layout_positions(layout, S, N, (r - s) % N), True, cu)
                for s in range(N)]
        assert got == want, (layout, varlen, r)


@pytest.mark.parametrize("layout,unit", [("zigzag_varlen", 8), ("stripe_varlen", 4)])
def test_step_pairs_per_sequence_layouts(bench_mod, ra, layout, unit):
    S, N = 512, 4
    cu = synth.cu_seqlens(synth.round_lengths(synth.loguniform_lengths(S, 16, 160, seed=5), unit))
    total = 0
    for r in range(N):
        got = bench_mod.step_pairs(ra, layout, S, N, r, cu)
        qpos = oracle.layout_positions(layout, S, N, r, cu)
        want = [oracle.count_pairs(qpos, oracle.layout_positions(layout, S, N, (r - s) % N, cu), True, cu)
                for s in range(N)]
        assert got == want, (layout, r)
        total += sum(got)
    # all ranks together see every causal pair of every sequence exactly once
    lengths = np.diff(np.asarray(cu, dtype=np.int64))
    assert total == int((lengths * (lengths + 1) // 2).sum())
