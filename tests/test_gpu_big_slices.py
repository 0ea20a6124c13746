"""Results whose (batch, head) slices pass 2 GiB: out, dQ and the other fp32
results are written through 64-bit addresses, so a block of 131328 query rows
x 32 heads x 128 dims (an fp32 slice of 2.004 GiB) is accepted and its rows
past the 2 GiB mark come out right.  Checked against the oracle on the first
and last rows (each row's out, lse and dQ depend on that row alone)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_grad, check_lse, check_out, dev, f64, log

pytestmark = pytest.mark.gpu


def test_block_fwd_bwd_rows_past_2gib():
    import torch
    import exact_long_context_ra_amd as ra
    B, H, D, LQ, LK = 1, 32, 128, 131328, 128
    log(f"big slices: lq={LQ} h={H} d={D} (fp32 slice {LQ * H * D * 4 / 2**30:.3f} GiB)")
    assert LQ * H * D * 4 > 2 ** 31
    q, do = synth.draw_normal([(B, LQ, H, D), (B, LQ, H, D)], torch.bfloat16, seed=51, device=dev())
    k, v = synth.draw_normal([(B, LK, H, D), (B, LK, H, D)], torch.bfloat16, seed=52, device=dev())
    # queries at positions LK .. LK + LQ - 1 see every key (causal over global positions)
    qm, km = ra.posmap([(LK, 1, LQ)]), ra.posmap([(0, 1, LK)])
    S = LK + LQ
    out, lse = ra.block_attn_fwd(q, k, v, qm, km, seq_len=S, causal=True)
    delta = ra.bwd_preprocess(out, do)
    dq = torch.zeros((B, LQ, H, D), device=dev(), dtype=torch.float32)
    dk = torch.zeros((B, LK, H, D), device=dev(), dtype=torch.float32)
    dv = torch.zeros((B, LK, H, D), device=dev(), dtype=torch.float32)
    ra.block_attn_bwd(q, k, v, do, lse, delta, qm, km, dq, dk, dv, seq_len=S, causal=True)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(64), np.arange(LQ - 192, LQ)])  # the last 192 lie past 2 GiB
    k64, v64 = f64(k), f64(v)
    q64, do64 = f64(q[:, rows]), f64(do[:, rows])
    qpos, kpos = LK + rows, np.arange(LK)
    ro, rl = oracle.attention(q64, k64, v64, qpos, kpos, True, None)
    gq, _, _ = oracle.attention_backward(q64, k64, v64, ro, rl, do64, qpos, kpos, True, None)
    check_out(f64(out[:, rows]), ro, True, what="out rows")
    check_lse(f64(lse[:, :, rows]), rl, True, what="lse rows")
    check_grad(f64(dq[:, rows]), gq, True, what="dq rows")
