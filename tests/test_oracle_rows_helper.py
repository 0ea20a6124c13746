"""The threaded row-block helper of the oracle (gpu_util.oracle_rows_fwd_bwd),
which the full-size GPU tests use to check whole heads, gives the same results
as one call of the oracle over the whole key set (it only hands each row block
the keys that block can see, and adds the blocks' dK/dV contributions)."""
import numpy as np
import pytest

import oracle
from gpu_util import oracle_rows_fwd_bwd


def _case(S, qpos, kpos, causal, cu, seed):
    rng = np.random.default_rng(seed)
    B, H, D = 1, 2, 16
    q = rng.standard_normal((B, len(qpos), H, D))
    k = rng.standard_normal((B, len(kpos), H, D))
    v = rng.standard_normal((B, len(kpos), H, D))
    do = rng.standard_normal((B, len(qpos), H, D))
    ro, rl = oracle.attention(q, k, v, qpos, kpos, causal, cu)
    gq, gk, gv = oracle.attention_backward(q, k, v, ro, rl, do, qpos, kpos, causal, cu)
    got = oracle_rows_fwd_bwd(q, k, v, do, qpos, kpos, causal, cu, block=7, workers=3)
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), got, (ro, rl, gq, gk, gv)):
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin), name
        assert np.allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12), name


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
@pytest.mark.parametrize("causal", [True, False])
def test_rows_helper_matches_oracle(layout, causal):
    S, N, r = 96, 4, 1
    _case(S, oracle.layout_positions(layout, S, N, r), np.arange(S), causal, None, seed=3)


@pytest.mark.parametrize("causal", [True, False])
def test_rows_helper_varlen(causal):
    S = 96
    cu = [0, 1, 20, 21, 60, 96]
    _case(S, np.arange(10, 70), np.arange(S), causal, cu, seed=4)
    # keys a strided subset of positions (a stripe block)
    _case(S, np.arange(1, S, 4), np.arange(3, S, 4), causal, cu, seed=5)
