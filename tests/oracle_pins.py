"""Checks that pin the float64 oracle to things other than itself.

Each ``check_*`` takes the oracle module (so that the mutation tests can hand
in a deliberately broken copy) and raises AssertionError on a mismatch.  The
references used here are: pure-Python brute force with no max shift, torch's
float64 scaled_dot_product_attention / logsumexp / autograd on the CPU, closed
forms, hand-derived values (tests/golden/hand_example.txt), values printed on
the pages (tests/golden/layout_examples.txt, ring_schedule.txt), integer
closed forms for per-rank work, and central finite differences.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        scale = max(1.0, float(np.max(np.abs(b[fin]))))
        assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol * scale:.3e}"


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# brute force (independent of the oracle's code)
# ---------------------------------------------------------------------------

def _brute_seq(p, cu):
    if cu is None:
        return 0
    for i in range(len(cu) - 1):
        if cu[i] <= p < cu[i + 1]:
            return i
    raise AssertionError("position outside cu_seqlens")


def brute_attention(q, k, v, qpos, kpos, causal, cu, scale):
    """Loops over every (row, key) pair; exp without any max shift."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    out = np.zeros((B, Lq, H, v.shape[3]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Lq):
                den = 0.0
                num = [0.0] * v.shape[3]
                for j in range(Lk):
                    if causal and not (kpos[j] <= qpos[i]):
                        continue
                    if _brute_seq(int(qpos[i]), cu) != _brute_seq(int(kpos[j]), cu):
                        continue
                    s = scale * sum(float(q[b, i, h, c]) * float(k[b, j, h, c]) for c in range(D))
                    w = math.exp(s)
                    den += w
                    for c in range(v.shape[3]):
                        num[c] += w * float(v[b, j, h, c])
                if den > 0:
                    lse[b, h, i] = math.log(den)
                    for c in range(v.shape[3]):
                        out[b, i, h, c] = num[c] / den
    return out, lse


def check_brute_force(orc):
    rng = np.random.default_rng(11)
    for causal, cu in [(False, None), (True, None), (True, [0, 3, 4, 9, 12]), (False, [0, 5, 12])]:
        B, Lq, Lk, H, D = 2, 5, 7, 2, 3
        q, k, v = _rand(rng, B, Lq, H, D), _rand(rng, B, Lk, H, D), _rand(rng, B, Lk, H, D)
        qpos = np.array(sorted(rng.choice(12, Lq, replace=False)))
        kpos = np.array(sorted(rng.choice(12, Lk, replace=False)))
        scale = 0.7
        o1, l1 = orc.attention(q, k, v, qpos, kpos, causal, cu, scale)
        o2, l2 = brute_attention(q, k, v, qpos, kpos, causal, cu, scale)
        _close(o1, o2, what=f"brute out causal={causal} cu={cu}")
        _close(l1, l2, what=f"brute lse causal={causal} cu={cu}")
    # default scale is 1/sqrt(d)
    q, k, v = _rand(rng, 1, 3, 1, 4), _rand(rng, 1, 4, 1, 4), _rand(rng, 1, 4, 1, 4)
    pos = np.arange(4)
    o1, l1 = orc.attention(q, k, v, pos[:3], pos, False)
    o2, l2 = brute_attention(q, k, v, pos[:3], pos, False, None, 0.5)
    _close(o1, o2, what="default-scale out")
    _close(l1, l2, what="default-scale lse")


# ---------------------------------------------------------------------------
# library routine: torch float64 SDPA and logsumexp on the CPU
# ---------------------------------------------------------------------------

def _torch_mask(qpos, kpos, causal, cu):
    import torch
    qp = torch.as_tensor(np.asarray(qpos))
    kp = torch.as_tensor(np.asarray(kpos))
    m = torch.ones(len(qp), len(kp), dtype=torch.bool)
    if causal:
        m &= kp[None, :] <= qp[:, None]
    if cu is not None:
        c = torch.as_tensor(np.asarray(cu))
        sq = torch.bucketize(qp, c, right=True) - 1
        sk = torch.bucketize(kp, c, right=True) - 1
        m &= sq[:, None] == sk[None, :]
    return m


def check_torch_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(12)
    cases = [
        ("contiguous", 64, 4, 1, False, None),
        ("zigzag", 64, 4, 2, True, None),
        ("stripe", 64, 4, 3, True, None),
        ("contiguous", 64, 4, 2, True, [0, 10, 11, 40, 64]),
    ]
    for layout, S, N, r, causal, cu in cases:
        B, H, D = 1, 2, 8
        qg, kg, vg = _rand(rng, B, S, H, D), _rand(rng, B, S, H, D), _rand(rng, B, S, H, D)
        qpos = orc.layout_positions(layout, S, N, r)
        kpos = np.arange(S)
        mask = _torch_mask(qpos, kpos, causal, cu)
        keep = mask.any(dim=1)
        tq = torch.from_numpy(qg[:, qpos]).permute(0, 2, 1, 3)
        tk = torch.from_numpy(kg).permute(0, 2, 1, 3)
        tv = torch.from_numpy(vg).permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(tq[:, :, keep], tk, tv, attn_mask=mask[keep], scale=0.3)
        sc = 0.3 * (tq @ tk.transpose(-1, -2))
        sc = sc.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=-1)
        o, l = orc.attention(qg[:, qpos], kg, vg, qpos, kpos, causal, cu, 0.3)
        _close(o[:, keep.numpy()], ref.permute(0, 2, 1, 3).numpy(), what=f"sdpa out {layout}")
        _close(l, ref_lse.numpy(), what=f"sdpa lse {layout}")


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def check_closed_forms(orc):
    rng = np.random.default_rng(13)
    B, S, H, D = 1, 24, 2, 5
    cu = [0, 7, 8, 24]
    pos = np.arange(S)
    q, k = _rand(rng, B, S, H, D), _rand(rng, B, S, H, D)
    vis = np.array([[(j <= i) and orc_free_same_seq(i, j, cu) for j in range(S)] for i in range(S)])
    nvis = vis.sum(axis=1)
    # (i) constant V gives V on every row with a visible key
    c = rng.standard_normal(D)
    vconst = np.broadcast_to(c, (B, S, H, D)).copy()
    o, _ = orc.attention(q, k, vconst, pos, pos, True, cu, 0.4)
    _close(o, vconst, what="constant V")
    # (ii) identical keys: mean of visible V, lse = s + ln|J|
    v = _rand(rng, B, S, H, D)
    kc = rng.standard_normal(D)
    kid = np.broadcast_to(kc, (B, S, H, D)).copy()
    o, l = orc.attention(q, kid, v, pos, pos, True, cu, 0.4)
    for i in range(S):
        J = np.nonzero(vis[i])[0]
        _close(o[:, i], v[:, J].mean(axis=1), what="identical keys out")
        _close(l[:, :, i], 0.4 * np.einsum("bhd,d->bh", q[:, i], kc) + math.log(len(J)),
               what="identical keys lse")
    # (iii) causal first token: O = v_0, lse = scale <q_0, k_0>
    o, l = orc.attention(q, k, v, pos, pos, True, None, 0.4)
    _close(o[:, 0], v[:, 0], what="first token out")
    _close(l[:, :, 0], 0.4 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), what="first token lse")
    # (iv) Q = 0: lse = ln|J|, O = mean of visible V
    o, l = orc.attention(np.zeros_like(q), k, v, pos, pos, True, cu, 0.4)
    for i in range(S):
        J = np.nonzero(vis[i])[0]
        _close(o[:, i], v[:, J].mean(axis=1), what="Q=0 out")
        _close(l[:, :, i], np.full((B, H), math.log(nvis[i])), what="Q=0 lse")
    # (v) a 1-token packed sequence attends only to itself (cu has [7, 8))
    _close(o[:, 7], v[:, 7], what="1-token sequence out")
    # (vi) no visible key: (0, -inf)
    o, l = orc.attention(q[:, :3], k[:, 10:], v[:, 10:], pos[:3], pos[10:], True)
    _close(o, np.zeros_like(o), what="empty rows out")
    assert np.all(np.isneginf(l)), "empty rows lse must be -inf"


def orc_free_same_seq(i, j, cu):
    return _brute_seq(i, cu) == _brute_seq(j, cu)


# ---------------------------------------------------------------------------
# hand-derived example
# ---------------------------------------------------------------------------

def load_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                parts = line.split()
                rows[parts[0]] = [float(x) for x in parts[1:]]
    return rows


def check_hand_example(orc):
    g = load_golden("hand_example.txt")
    q = np.array(g["q"]).reshape(1, 1, 1, 2)
    k = np.array([g["k0"], g["k1"]]).reshape(1, 2, 1, 2)
    v = np.array([g["v0"], g["v1"]]).reshape(1, 2, 1, 2)
    kpos = np.array([0, 1])
    o, l = orc.attention(q, k, v, np.array([1]), kpos, False)
    _close(o.ravel(), g["out"], what="hand out")
    _close(l.ravel(), g["lse"], what="hand lse")
    o, l = orc.attention(q, k, v, np.array([0]), kpos, True)
    _close(o.ravel(), g["out_causal_q0"], what="hand causal out")
    _close(l.ravel(), g["lse_causal_q0"], what="hand causal lse")
    o0, l0 = orc.attention(q, k[:, :1], v[:, :1], np.array([1]), kpos[:1], False)
    o1, l1 = orc.attention(q, k[:, 1:], v[:, 1:], np.array([1]), kpos[1:], False)
    _close(np.concatenate([o0.ravel(), l0.ravel()]), g["block0"], what="hand block0")
    _close(np.concatenate([o1.ravel(), l1.ravel()]), g["block1"], what="hand block1")
    om, lm = orc.lse_merge(o0, l0, o1, l1)
    _close(om.ravel(), g["out"], what="hand merged out")
    _close(lm.ravel(), g["lse"], what="hand merged lse")
    o, l = orc.attention(q, k, v, np.array([1]), kpos, False)
    do = np.array(g["dout"]).reshape(1, 1, 1, 2)
    dq, dk, dv = orc.attention_backward(q, k, v, o, l, do, np.array([1]), kpos, False)
    _close(dq.ravel(), g["dq"], what="hand dq")
    _close(dk[0, 0, 0], g["dk0"], what="hand dk0")
    _close(dk[0, 1, 0], g["dk1"], what="hand dk1")
    _close(dv[0, 0, 0], g["dv0"], what="hand dv0")
    _close(dv[0, 1, 0], g["dv1"], what="hand dv1")


# ---------------------------------------------------------------------------
# block decomposition: merging block results over any split is one-shot softmax
# ---------------------------------------------------------------------------

def check_split_merge(orc):
    rng = np.random.default_rng(14)
    B, Lq, Lk, H, D = 2, 9, 23, 2, 4
    for trial in range(6):
        causal = trial % 2 == 0
        cu = [0, 4, 5, 30] if trial >= 4 else None
        q, k, v = _rand(rng, B, Lq, H, D, scale=2.0), _rand(rng, B, Lk, H, D), _rand(rng, B, Lk, H, D)
        qpos = np.sort(rng.choice(30, Lq, replace=False))
        kpos = np.sort(rng.choice(30, Lk, replace=False))
        full = orc.attention(q, k, v, qpos, kpos, causal, cu)
        # random partition into blocks, including empty and singleton blocks, random order
        labels = rng.integers(0, 6, Lk)
        labels[0] = 5  # singleton candidate
        order = rng.permutation(7)  # block 6 is always empty
        parts = []
        for blk in order:
            idx = np.nonzero(labels == blk)[0]
            parts.append(orc.attention(q, k[:, idx], v[:, idx], qpos, kpos[idx], causal, cu))
        got = orc.merge_all(parts, full[0].shape, full[1].shape)
        _close(got[0], full[0], what=f"split/merge out trial {trial}")
        _close(got[1], full[1], what=f"split/merge lse trial {trial}")
    # merging with an empty side is the identity
    o, l = full
    e_o, e_l = np.zeros_like(o), np.full_like(l, -np.inf)
    for a, b in [((o, l), (e_o, e_l)), ((e_o, e_l), (o, l))]:
        m = orc.lse_merge(*a, *b)
        _close(m[0], o, what="merge identity out")
        _close(m[1], l, what="merge identity lse")


# ---------------------------------------------------------------------------
# layouts: values printed on the pages, permutation, closed-form work per rank
# ---------------------------------------------------------------------------

def check_layout_golden(orc):
    with open(os.path.join(GOLDEN, "layout_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            layout, S, N, r = parts[0], int(parts[1]), int(parts[2]), int(parts[3])
            pos = orc.layout_positions(layout, S, N, r)
            for item in parts[4:]:
                a, p = item.split(":")
                assert int(pos[int(a)]) == int(p), f"{layout} r={r} local {a}: {pos[int(a)]} != {p}"
    with open(os.path.join(GOLDEN, "ring_schedule.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            vals = [int(x) for x in line.split()]
            N, r, srcs = vals[0], vals[1], vals[2:]
            assert list(orc.ring_sources(N, r)) == srcs, f"schedule N={N} r={r}"


def closed_form_pairs(layout, S, N, r):
    """Causal pairs of rank r's queries over the whole sequence.

    A query at global position p sees exactly p+1 keys, so the count is the
    sum of (p+1) over the rank's positions, which in closed form is:
      contiguous (L = S/N):  r L^2 + L(L+1)/2
      zigzag (C = S/2N):     2N C^2 + C            (the same for every rank)
      stripe (L = S/N):      N L(L-1)/2 + (r+1) L
    """
    if layout == "contiguous":
        L = S // N
        return r * L * L + L * (L + 1) // 2
    if layout == "zigzag":
        C = S // (2 * N)
        return 2 * N * C * C + C
    if layout == "stripe":
        L = S // N
        return N * L * (L - 1) // 2 + (r + 1) * L
    raise ValueError(layout)


def check_layouts(orc):
    for layout in ("contiguous", "zigzag", "stripe"):
        for S, N in [(16, 1), (16, 2), (24, 3), (64, 4), (128, 8)]:
            allpos = np.concatenate([orc.layout_positions(layout, S, N, r) for r in range(N)])
            assert np.array_equal(np.sort(allpos), np.arange(S)), f"{layout} S={S} N={N} not a permutation"
            tot = 0
            for r in range(N):
                qpos = orc.layout_positions(layout, S, N, r)
                assert np.all(np.diff(qpos) > 0), "local order must follow global order"
                got = sum(orc.count_pairs(qpos, orc.layout_positions(layout, S, N, src), True)
                          for src in range(N))
                assert got == closed_form_pairs(layout, S, N, r), f"{layout} S={S} N={N} r={r} pairs {got}"
                tot += got
            assert tot == S * (S + 1) // 2
    # zigzag balances causal work exactly across ranks
    vals = {closed_form_pairs("zigzag", 256, 8, r) for r in range(8)}
    assert len(vals) == 1


def check_varlen_layout_golden(orc):
    with open(os.path.join(GOLDEN, "varlen_layout_examples.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            layout, S, N, r = parts[0], int(parts[1]), int(parts[2]), int(parts[3])
            cu = [int(x) for x in parts[4].split(",")]
            want = [int(x) for x in parts[5:]]
            got = orc.layout_positions(layout, S, N, r, cu)
            assert list(got) == want, f"{layout} S={S} N={N} r={r} cu={cu}: {list(got)}"


def check_varlen_layouts(orc):
    """Per-sequence layouts: a permutation of the stream; with one sequence the
    plain layout; each rank's tokens of a sequence stay inside it, in order;
    causal pair counts per rank equal the per-sequence closed forms summed,
    and zigzag keeps them equal across ranks."""
    for base, mult in (("zigzag", 2), ("stripe", 1)):
        layout = base + "_varlen"
        for N in (1, 2, 3, 4):
            S = 8 * mult * N
            for r in range(N):
                assert np.array_equal(orc.layout_positions(layout, S, N, r, [0, S]),
                                      orc.layout_positions(base, S, N, r))
            for cu in ([0, S], [0, mult * N, S], [0, mult * N * 3, mult * N * 3, S],
                       [0, mult * N, 2 * mult * N, 5 * mult * N, S]):
                allpos = np.concatenate([orc.layout_positions(layout, S, N, r, cu) for r in range(N)])
                assert np.array_equal(np.sort(allpos), np.arange(S)), f"{layout} {cu} not a permutation"
                counts = []
                for r in range(N):
                    qpos = orc.layout_positions(layout, S, N, r, cu)
                    assert np.all(np.diff(qpos) > 0), "local order must follow global order"
                    sid = np.searchsorted(cu, qpos, side="right") - 1
                    per = np.bincount(sid, minlength=len(cu) - 1)
                    assert np.array_equal(per, np.diff(cu) // N), f"{layout} {cu} r={r}: tokens per sequence"
                    got = sum(orc.count_pairs(qpos, orc.layout_positions(layout, S, N, src, cu), True, cu)
                              for src in range(N))
                    want = sum(closed_form_pairs(base, n, N, r) for n in np.diff(cu) if n > 0)
                    assert got == want, f"{layout} {cu} r={r}: pairs {got} != {want}"
                    counts.append(got)
                if base == "zigzag":
                    assert len(set(counts)) == 1, f"zigzag_varlen {cu}: unbalanced {counts}"


def check_stripe_rule(orc):
    """Stripe step mask in local indices: key b visible to query a iff
    b <= a when src <= r, and b <= a-1 when src > r (from pos = index*N + rank)."""
    for S, N in [(24, 3), (32, 4), (40, 8)]:
        L = S // N
        a = np.arange(L)[:, None]
        b = np.arange(L)[None, :]
        for r in range(N):
            for src in range(N):
                m = orc.visible(orc.layout_positions("stripe", S, N, r),
                                orc.layout_positions("stripe", S, N, src), True)
                rule = (b <= a) if src <= r else (b <= a - 1)
                assert np.array_equal(m, rule), f"stripe rule S={S} N={N} r={r} src={src}"


# ---------------------------------------------------------------------------
# the ring reaches full attention
# ---------------------------------------------------------------------------

def check_ring_union(orc):
    rng = np.random.default_rng(15)
    B, H, D = 1, 2, 6
    for layout, S, N, causal, cu in [
        ("contiguous", 32, 4, True, None), ("zigzag", 32, 4, True, None),
        ("stripe", 32, 4, True, None), ("contiguous", 24, 3, False, None),
        ("zigzag", 48, 3, True, None), ("stripe", 24, 2, False, None),
        ("contiguous", 32, 4, True, [0, 5, 6, 19, 32]),
        ("stripe", 32, 4, True, [0, 9, 32]),
        ("zigzag_varlen", 48, 3, True, [0, 6, 6, 30, 48]),
        ("stripe_varlen", 36, 4, True, [0, 4, 24, 36]),
    ]:
        qg, kg, vg = _rand(rng, B, S, H, D), _rand(rng, B, S, H, D), _rand(rng, B, S, H, D)
        full_o, full_l = brute_attention(qg, kg, vg, np.arange(S), np.arange(S), causal, cu,
                                         1 / math.sqrt(D))
        kr, vr = orc.to_ring(kg, layout, N, cu), orc.to_ring(vg, layout, N, cu)
        got_o = np.zeros_like(full_o)
        got_l = np.zeros_like(full_l)
        for r in range(N):
            pos = orc.layout_positions(layout, S, N, r, cu)
            o, l = orc.ring_forward(layout, N, r, qg[:, pos], kr, vr, causal, cu)
            got_o[:, pos] = o
            got_l[:, :, pos] = l
        _close(got_o, full_o, what=f"ring union out {layout} N={N} cu={cu}")
        _close(got_l, full_l, what=f"ring union lse {layout} N={N} cu={cu}")
        # resume: steps [0, s) then [s, N) equals all steps
        r = N - 1
        pos = orc.layout_positions(layout, S, N, r, cu)
        s = N // 2
        first = orc.ring_forward(layout, N, r, qg[:, pos], kr, vr, causal, cu, steps=range(s))
        second = orc.ring_forward(layout, N, r, qg[:, pos], kr, vr, causal, cu,
                                  steps=range(s, N), init=first)
        _close(second[0], full_o[:, pos], what="resume out")
        _close(second[1], full_l[:, :, pos], what="resume lse")


def check_varlen_independent(orc):
    rng = np.random.default_rng(16)
    lengths = [5, 1, 9, 3, 14]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    S = int(cu[-1])
    B, H, D = 1, 2, 4
    q, k, v = _rand(rng, B, S, H, D), _rand(rng, B, S, H, D), _rand(rng, B, S, H, D)
    pos = np.arange(S)
    for causal in (True, False):
        o, l = orc.attention(q, k, v, pos, pos, causal, cu)
        for a, b in zip(cu[:-1], cu[1:]):
            seg = np.arange(a, b)
            so, sl = brute_attention(q[:, seg], k[:, seg], v[:, seg], seg - a, seg - a, causal, None,
                                     1 / math.sqrt(D))
            _close(o[:, seg], so, what="varlen seq out")
            _close(l[:, :, seg], sl, what="varlen seq lse")
    # the 1-token sequence: O = v, lse = scale <q, k>
    i = 5
    o, l = orc.attention(q, k, v, pos, pos, True, cu)
    _close(o[:, i], v[:, i], what="1-token out")
    _close(l[:, :, i], np.einsum("bhd,bhd->bh", q[:, i], k[:, i]) / math.sqrt(D), what="1-token lse")


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def check_backward_fd(orc):
    """Central finite differences of F = sum(dO * O) in float64."""
    rng = np.random.default_rng(17)
    B, L, H, D = 1, 5, 1, 3
    q, k, v, do = (_rand(rng, B, L, H, D) for _ in range(4))
    qpos = np.array([2, 4, 5, 7, 9])
    kpos = np.array([0, 3, 4, 8, 9])
    cu = [0, 6, 10]
    for causal in (True, False):
        o, l = orc.attention(q, k, v, qpos, kpos, causal, cu)
        dq, dk, dv = orc.attention_backward(q, k, v, o, l, do, qpos, kpos, causal, cu)
        hstep = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += hstep
                xm[idx] -= hstep
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                fp = np.sum(do * orc.attention(args_p["q"], args_p["k"], args_p["v"], qpos, kpos, causal, cu)[0])
                fm = np.sum(do * orc.attention(args_m["q"], args_m["k"], args_m["v"], qpos, kpos, causal, cu)[0])
                num[idx] = (fp - fm) / (2 * hstep)
            err = np.max(np.abs(num - g))
            assert err <= 1e-7 * max(1.0, np.max(np.abs(g))), f"FD d{name} causal={causal}: {err:.3e}"


def check_backward_autograd(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(18)
    B, S, H, D = 1, 40, 2, 8
    cu = [0, 13, 14, 40]
    for causal, cuv in [(True, None), (True, cu), (False, None)]:
        q, k, v, do = (_rand(rng, B, S, H, D) for _ in range(4))
        pos = np.arange(S)
        o, l = orc.attention(q, k, v, pos, pos, causal, cuv)
        dq, dk, dv = orc.attention_backward(q, k, v, o, l, do, pos, pos, causal, cuv)
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
        mask = _torch_mask(pos, pos, causal, cuv)
        out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
        _close(dq, tq.grad.permute(0, 2, 1, 3).numpy(), tol=1e-11, what="autograd dq")
        _close(dk, tk.grad.permute(0, 2, 1, 3).numpy(), tol=1e-11, what="autograd dk")
        _close(dv, tv.grad.permute(0, 2, 1, 3).numpy(), tol=1e-11, what="autograd dv")


def check_backward_invariants(orc):
    rng = np.random.default_rng(19)
    B, S, H, D = 1, 30, 2, 5
    cu = [0, 12, 13, 30]
    pos = np.arange(S)
    q, k, v, do = (_rand(rng, B, S, H, D) for _ in range(4))
    o, l = orc.attention(q, k, v, pos, pos, True, cu)
    dq, dk, dv = orc.attention_backward(q, k, v, o, l, do, pos, pos, True, cu)
    # each row of dS sums to zero -> sum_j dK_j = 0
    _close(dk.sum(axis=1), np.zeros((B, H, D)), tol=1e-12, what="sum dK")
    # each row of P sums to one -> sum_j dV_j = sum_i dO_i
    _close(dv.sum(axis=1), do.sum(axis=1), tol=1e-12, what="sum dV")
    # constant V -> dQ = dK = 0
    vc = np.broadcast_to(rng.standard_normal(D), v.shape).copy()
    o2, l2 = orc.attention(q, k, vc, pos, pos, True, cu)
    dq2, dk2, _ = orc.attention_backward(q, k, vc, o2, l2, do, pos, pos, True, cu)
    _close(dq2, np.zeros_like(dq2), what="const V dQ")
    _close(dk2, np.zeros_like(dk2), what="const V dK")
    # identical keys -> dQ = 0
    kc = np.broadcast_to(rng.standard_normal(D), k.shape).copy()
    o3, l3 = orc.attention(q, kc, v, pos, pos, True, cu)
    dq3, _, _ = orc.attention_backward(q, kc, v, o3, l3, do, pos, pos, True, cu)
    _close(dq3, np.zeros_like(dq3), what="identical keys dQ")


def check_ring_backward_union(orc):
    rng = np.random.default_rng(20)
    B, H, D = 1, 2, 4
    for layout, S, N, cu in [("contiguous", 24, 3, None), ("zigzag", 32, 4, None),
                             ("stripe", 24, 4, None), ("contiguous", 32, 4, [0, 3, 20, 32]),
                             ("zigzag_varlen", 36, 3, [0, 12, 12, 36]),
                             ("stripe_varlen", 28, 4, [0, 8, 28])]:
        qg, kg, vg, dog = (_rand(rng, B, S, H, D) for _ in range(4))
        pos = np.arange(S)
        fo, fl = orc.attention(qg, kg, vg, pos, pos, True, cu)
        fdq, fdk, fdv = orc.attention_backward(qg, kg, vg, fo, fl, dog, pos, pos, True, cu)
        kr, vr = orc.to_ring(kg, layout, N, cu), orc.to_ring(vg, layout, N, cu)
        dk_sum = np.zeros_like(kr)
        dv_sum = np.zeros_like(vr)
        for r in range(N):
            p = orc.layout_positions(layout, S, N, r, cu)
            o, l = orc.ring_forward(layout, N, r, qg[:, p], kr, vr, True, cu)
            dq, dkr, dvr = orc.ring_backward(layout, N, r, qg[:, p], kr, vr, o, l, dog[:, p], True, cu)
            _close(dq, fdq[:, p], what=f"ring bwd dq {layout}")
            dk_sum += dkr
            dv_sum += dvr
        _close(dk_sum, orc.to_ring(fdk, layout, N, cu), what=f"ring bwd dk {layout}")
        _close(dv_sum, orc.to_ring(fdv, layout, N, cu), what=f"ring bwd dv {layout}")


ALL_CHECKS = [
    check_brute_force, check_torch_sdpa, check_closed_forms, check_hand_example,
    check_split_merge, check_layout_golden, check_layouts, check_varlen_layout_golden,
    check_varlen_layouts, check_stripe_rule,
    check_ring_union, check_varlen_independent, check_backward_fd,
    check_backward_autograd, check_backward_invariants, check_ring_backward_union,
]
