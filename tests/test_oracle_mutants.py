"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them: a pin set that a dropped term, a wrong sign
or index, or a transposed operand slips through would prove nothing."""
import importlib.util
import os

import pytest

import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "ring_attention.py")

MUTANTS = {
    "scale_1_over_d": ("return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    "causal_strict": ("ok &= kpos[None, :] <= qpos[:, None]", "ok &= kpos[None, :] < qpos[:, None]"),
    "no_seq_mask": ("ok &= seq_ids(qpos, cu_seqlens)[:, None] == seq_ids(kpos, cu_seqlens)[None, :]",
                    "pass"),
    "lse_log2": ("m + np.log(np.where(has, l, 1.0))", "m + np.log2(np.where(has, l, 1.0))"),
    "pv_uses_k": ("out[b, i0:i1, h, :] = p @ v[b, :, h, :]", "out[b, i0:i1, h, :] = p @ k[b, :, h, :]"),
    "merge_sign": ("np.exp(lse_b - m_safe))", "np.exp(m_safe - lse_b))"),
    "merge_no_renorm": ("l_safe = np.where(empty, 1.0, l_new)", "l_safe = np.where(empty, 1.0, 1.0)"),
    "zigzag_pair": ("j = 2 * N - 1 - r", "j = 2 * N - 2 - r"),
    "stripe_offset": ("return np.arange(r, S, N, dtype=np.int64)",
                      "return np.arange(r * (S // N), S, 1, dtype=np.int64)[: S // N]"),
    "ring_direction": ("return [(rank - s) % world for s in range(world)]",
                       "return [(rank + s) % world for s in range(world)]"),
    "bwd_drop_delta": ("ds = p * (dp - delta[b, h, i0:i1][:, None])", "ds = p * dp"),
    "bwd_dk_uses_k": ("dk[b, :, h, :] += scale * (ds.T @ q[b, i0:i1, h, :])",
                      "dk[b, :, h, :] += scale * (ds.T @ k[b, i0:i1, h, :])"),
    "bwd_dq_no_scale": ("dq[b, i0:i1, h, :] = scale * (ds @ k[b, :, h, :])",
                        "dq[b, i0:i1, h, :] = ds @ k[b, :, h, :]"),
    "bwd_dv_uses_ds": ("dv[b, :, h, :] += p.T @ do", "dv[b, :, h, :] += ds.T @ do"),
    "varlen_layout_no_offset": ("parts = [cu[i] + layout_positions(base",
                                "parts = [0 * cu[i] + layout_positions(base"),
    "varlen_layout_whole_stream": ("base = layout[: -len(\"_varlen\")]",
                                   "return layout_positions(layout[: -len(\"_varlen\")], S, N, r)"),
    "bwd_p_uses_m": ("np.exp(s - np.where(live, row_lse, 0.0)[:, None]), 0.0)",
                     "np.exp(s - np.where(live, row_lse + 0.5, 0.0)[:, None]), 0.0)"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not unique/found"
    text = text.replace(old, new)
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _load_mutant(name)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"
