"""Float64 CPU oracle for Ring Attention's per-device computation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and
by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares no
code with the HIP library (no kernels, headers, helpers or tables); the only
thing both sides consume is the seeded input generator in ``synth/``.

Sources (the pages this oracle is written from):

* [RFA]  "Ring Flash Attention" README (github.com/zhuzilin/ring-flash-attention):
  the function list (ring / zigzag ring / stripe, stripe = block size 1), the
  statement that each block's ``softmax_lse`` is what lets block results be
  combined, the single ``cu_seqlens`` restriction of the varlen forms, and the
  "Limits" section (bf16 per-block outputs cause accumulation error).
* [BLOG] "Ring Attention：突破百万 Token 上下文的分布式注意力" (guijiagi.com):
  section "详细流程" (ring schedule: at iteration t device i works on the K/V
  block of device i-(t-1)), the plain PyTorch ``ring_attention`` listing
  (scores scaled by 1/sqrt(d), online-softmax state (max, exp-sum), final
  division), section "在线 Softmax：关键技巧" (the (m, l) update), and section
  "Striped Ring Attention" (token t lives on device t mod N).
* [NEWS] ainews.cool article, section "技术深度解析": S = QK^T, tiles, each
  device keeps its local Q block and receives K/V blocks around the ring; the
  global output is the concatenation of the devices' outputs.
* [STRIPE] briefgpt.xyz abstract of "Striped Attention: Faster Ring Attention
  for Causal Transformers": causal masking makes contiguous shards unbalanced;
  striping tokens uniformly over devices rebalances them.

Readings taken where the pages are silent or garbled (each is also listed in
the design notes):

* softmax_lse is the natural log of the sum of exp(scaled score) over the
  allowed keys of a row; a row with no allowed key has (out, lse) = (0, -inf).
* Zigzag: the sequence is cut into 2N equal chunks and rank r holds chunks r
  and 2N-1-r, in that order (the blog's zigzag example is incomplete).
* Masks are evaluated on GLOBAL token positions: key j is visible to query i
  iff (not causal or pos_k(j) <= pos_q(i)) and both lie in the same packed
  sequence of ``cu_seqlens`` (one array shared by q and k/v, [RFA]).
* The block step of the ring uses the K/V block of rank src = (r - s) mod N at
  step s; the result does not depend on the order (only rounding does).
* The backward is the textbook gradient of softmax attention (the pages give
  no backward); P is recomputed from the final lse and D_i = <dO_i, O_i>.

Array conventions: token-major ``[batch, tokens, heads, head_dim]`` for q, k, v,
out, dout, dq, dk, dv; ``[batch, heads, tokens]`` for lse; positions are int64
vectors over the local token axis.  All arithmetic is float64.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

LAYOUTS = ("contiguous", "zigzag", "stripe", "zigzag_varlen", "stripe_varlen")

# Work per row-block of the score matrix: at most this many float64 scores.
_BLOCK_ELEMS = 1 << 24


# ---------------------------------------------------------------------------
# Token-to-device layouts  ([BLOG] "详细流程" and "Striped Ring Attention";
# [RFA] function list; [STRIPE] abstract)
# ---------------------------------------------------------------------------

def layout_positions(layout: str, seq_len: int, world: int, rank: int, cu_seqlens=None) -> np.ndarray:
    """Global token position of each local token of ``rank`` (local order).

    contiguous: rank r owns the r-th of N equal consecutive chunks.
    zigzag:     2N equal chunks; rank r owns chunk r then chunk 2N-1-r.
    stripe:     token t belongs to rank t mod N (a "block size" of one token).
    zigzag_varlen / stripe_varlen: the same layout applied to every packed
        sequence of ``cu_seqlens`` on its own ([RFA] function list: the zigzag
        and stripe forms of the varlen function); rank r's tokens are its part
        of sequence 0, then its part of sequence 1, and so on.  Every sequence
        length must split evenly (2N chunks for zigzag, N for stripe).
    ``cu_seqlens`` is used by the per-sequence layouts only.
    """
    S, N, r = int(seq_len), int(world), int(rank)
    if not (0 <= r < N):
        raise ValueError("rank out of range")
    if layout in ("zigzag_varlen", "stripe_varlen"):
        if cu_seqlens is None:
            raise ValueError(f"{layout} needs cu_seqlens")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu[0] != 0 or cu[-1] != S or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must rise from 0 to seq_len")
        base = layout[: -len("_varlen")]
        parts = [cu[i] + layout_positions(base, int(cu[i + 1] - cu[i]), N, r) for i in range(len(cu) - 1)]
        return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    if layout == "contiguous":
        if S % N:
            raise ValueError("seq_len must be divisible by world")
        L = S // N
        return np.arange(r * L, (r + 1) * L, dtype=np.int64)
    if layout == "zigzag":
        if S % (2 * N):
            raise ValueError("seq_len must be divisible by 2*world")
        C = S // (2 * N)
        first = np.arange(r * C, (r + 1) * C, dtype=np.int64)
        j = 2 * N - 1 - r
        second = np.arange(j * C, (j + 1) * C, dtype=np.int64)
        return np.concatenate([first, second])
    if layout == "stripe":
        if S % N:
            raise ValueError("seq_len must be divisible by world")
        return np.arange(r, S, N, dtype=np.int64)
    raise ValueError(f"unknown layout {layout!r}")


def ring_sources(world: int, rank: int) -> List[int]:
    """Rank whose K/V block ``rank`` works on at each ring step.

    [BLOG] "详细流程": iteration 1 uses the device's own block, iteration 2 the
    block of device i-1, iteration 3 that of device i-2, and so on, modulo N.
    """
    return [(rank - s) % world for s in range(world)]


# ---------------------------------------------------------------------------
# Visibility of keys to queries
# ---------------------------------------------------------------------------

def seq_ids(pos: np.ndarray, cu_seqlens: Optional[Sequence[int]]) -> np.ndarray:
    """Index of the packed sequence holding each global position (0 if none)."""
    pos = np.asarray(pos, dtype=np.int64)
    if cu_seqlens is None:
        return np.zeros(pos.shape, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    if pos.size and (pos.min() < 0 or pos.max() >= cu[-1]):
        raise ValueError("position outside cu_seqlens range")
    return np.searchsorted(cu, pos, side="right") - 1


def visible(qpos: np.ndarray, kpos: np.ndarray, causal: bool,
            cu_seqlens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [Lq, Lk]: may query i attend to key j (global positions)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    ok = np.ones((qpos.size, kpos.size), dtype=bool)
    if causal:
        ok &= kpos[None, :] <= qpos[:, None]
    if cu_seqlens is not None:
        ok &= seq_ids(qpos, cu_seqlens)[:, None] == seq_ids(kpos, cu_seqlens)[None, :]
    return ok


def count_pairs(qpos, kpos, causal: bool, cu_seqlens=None) -> int:
    """Number of visible (query, key) pairs, counted from the mask itself."""
    qpos = np.asarray(qpos, dtype=np.int64)
    total = 0
    step = max(1, _BLOCK_ELEMS // max(1, len(kpos)))
    for i0 in range(0, qpos.size, step):
        total += int(visible(qpos[i0:i0 + step], kpos, causal, cu_seqlens).sum())
    return total


def default_scale(head_dim: int) -> float:
    """Scores are scaled by 1/sqrt(d) ([BLOG] ring_attention listing)."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# Exact softmax attention (the plain definition the ring reaches exactly)
# ---------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, qpos, kpos, causal: bool = False, cu_seqlens=None,
              scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of q over the visible keys of (k, v).

    Per query row i with visible set J_i and scores s_ij = scale*<q_i, k_j>:
      m_i   = max_J s_ij
      lse_i = m_i + ln sum_J exp(s_ij - m_i)
      out_i = sum_J exp(s_ij - lse_i) v_j
    and (out_i, lse_i) = (0, -inf) when J_i is empty.
    Returns out [b, Lq, h, d] and lse [b, h, Lq].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, H, Dh = q.shape
    Lk = k.shape[1]
    if scale is None:
        scale = default_scale(Dh)
    out = np.zeros((B, Lq, H, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, Lq), -np.inf, dtype=np.float64)
    if Lq == 0 or Lk == 0:
        return out, lse
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    step = max(1, _BLOCK_ELEMS // Lk)
    for i0 in range(0, Lq, step):
        i1 = min(Lq, i0 + step)
        mask = visible(qpos[i0:i1], kpos, causal, cu_seqlens)
        has = mask.any(axis=1)
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, i0:i1, h, :] @ k[b, :, h, :].T)
                s = np.where(mask, s, -np.inf)
                m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
                l = np.exp(s - m[:, None]).sum(axis=1)
                row_lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
                p = np.where(has[:, None], np.exp(s - np.where(has, row_lse, 0.0)[:, None]), 0.0)
                out[b, i0:i1, h, :] = p @ v[b, :, h, :]
                lse[b, h, i0:i1] = row_lse
    return out, lse


# ---------------------------------------------------------------------------
# Combining block results through their softmax_lse
# ([RFA] main idea; [BLOG] "在线 Softmax：关键技巧")
# ---------------------------------------------------------------------------

def lse_merge(out, lse, out_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Fold a block result (out_b, lse_b) into a running result (out, lse).

    Each input is a softmax-normalised partial output together with its
    log-sum-exp.  Writing each as the blog's online-softmax state
    (m, l) = (lse, 1) and applying its update:
      m_new = max(m_old, m_blk)
      l_new = l_old*exp(m_old - m_new) + l_blk*exp(m_blk - m_new)
      out   = (out_old*l_old*exp(m_old - m_new) + out_blk*l_blk*exp(m_blk - m_new)) / l_new
    and returning lse_new = m_new + ln l_new.  A side whose lse is -inf holds
    no keys and contributes nothing.
    out: [b, L, h, d]; lse: [b, h, L].
    """
    out, lse, out_b, lse_b = _f64(out), _f64(lse), _f64(out_b), _f64(lse_b)
    m_new = np.maximum(lse, lse_b)
    empty = np.isneginf(m_new)
    m_safe = np.where(empty, 0.0, m_new)
    w_old = np.where(np.isneginf(lse), 0.0, np.exp(lse - m_safe))
    w_blk = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    l_new = w_old + w_blk
    l_safe = np.where(empty, 1.0, l_new)
    # [b, h, L] weights -> [b, L, h, 1] to scale the token-major outputs
    a_old = np.transpose(w_old / l_safe, (0, 2, 1))[..., None]
    a_blk = np.transpose(w_blk / l_safe, (0, 2, 1))[..., None]
    out_new = a_old * out + a_blk * out_b
    lse_new = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return out_new, lse_new


def merge_all(parts: Iterable[Tuple[np.ndarray, np.ndarray]], shape_out, shape_lse):
    """Left fold of ``lse_merge`` starting from the empty result (0, -inf)."""
    out = np.zeros(shape_out, dtype=np.float64)
    lse = np.full(shape_lse, -np.inf, dtype=np.float64)
    for o, l in parts:
        out, lse = lse_merge(out, lse, o, l)
    return out, lse


# ---------------------------------------------------------------------------
# The virtual ring: one rank's share, all steps run one after another
# ---------------------------------------------------------------------------

def ring_forward(layout: str, world: int, rank: int, q_local, k_ring, v_ring,
                 causal: bool = True, cu_seqlens=None, scale: Optional[float] = None,
                 steps: Optional[Sequence[int]] = None, init=None):
    """Forward of ``rank``'s share: q_local [b, L, h, d] against every block.

    k_ring/v_ring: [N, b, L, h, d], block n being rank n's local K/V in its
    layout order.  At step s the block of src = (rank - s) mod N is attended
    (attention restricted to that block, masked on global positions) and the
    result is merged into the running (out, lse).  ``steps`` selects a subset
    of steps (default: all N) and ``init`` resumes from a previous state.
    Returns out [b, L, h, d], lse [b, h, L].
    """
    q_local = _f64(q_local)
    B, L, H, Dh = q_local.shape
    S = L * world
    qpos = layout_positions(layout, S, world, rank, cu_seqlens)
    srcs = ring_sources(world, rank)
    if steps is None:
        steps = range(world)
    if init is None:
        out = np.zeros((B, L, H, v_ring.shape[-1]), dtype=np.float64)
        lse = np.full((B, H, L), -np.inf, dtype=np.float64)
    else:
        out, lse = _f64(init[0]).copy(), _f64(init[1]).copy()
    for s in steps:
        src = srcs[s]
        kpos = layout_positions(layout, S, world, src, cu_seqlens)
        ob, lb = attention(q_local, k_ring[src], v_ring[src], qpos, kpos, causal, cu_seqlens, scale)
        out, lse = lse_merge(out, lse, ob, lb)
    return out, lse


# ---------------------------------------------------------------------------
# Backward (textbook softmax-attention gradient; not given on the pages)
# ---------------------------------------------------------------------------

def attention_backward(q, k, v, out, lse, dout, qpos, kpos, causal: bool = False,
                       cu_seqlens=None, scale: Optional[float] = None):
    """Gradients of attention restricted to the keys (k, v) with FINAL (out, lse).

    With P_ij = exp(s_ij - lse_i) on visible pairs (0 elsewhere) and
    D_i = <dO_i, O_i>:
      dV_j = sum_i P_ij dO_i
      dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)
      dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
    When (k, v) is the whole key set these are the exact gradients of
    sum(dout * out); for a subset they are that block's share of them.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    out, lse, dout = _f64(out), _f64(lse), _f64(dout)
    B, Lq, H, Dh = q.shape
    Lk = k.shape[1]
    if scale is None:
        scale = default_scale(Dh)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Lq == 0 or Lk == 0:
        return dq, dk, dv
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    delta = np.einsum("blhd,blhd->bhl", dout, out)
    step = max(1, _BLOCK_ELEMS // Lk)
    for i0 in range(0, Lq, step):
        i1 = min(Lq, i0 + step)
        mask = visible(qpos[i0:i1], kpos, causal, cu_seqlens)
        for b in range(B):
            for h in range(H):
                row_lse = lse[b, h, i0:i1]
                live = ~np.isneginf(row_lse)
                s = scale * (q[b, i0:i1, h, :] @ k[b, :, h, :].T)
                p = np.where(mask & live[:, None],
                             np.exp(s - np.where(live, row_lse, 0.0)[:, None]), 0.0)
                do = dout[b, i0:i1, h, :]
                dp = do @ v[b, :, h, :].T
                ds = p * (dp - delta[b, h, i0:i1][:, None])
                dq[b, i0:i1, h, :] = scale * (ds @ k[b, :, h, :])
                dk[b, :, h, :] += scale * (ds.T @ q[b, i0:i1, h, :])
                dv[b, :, h, :] += p.T @ do
    return dq, dk, dv


def ring_backward(layout: str, world: int, rank: int, q_local, k_ring, v_ring,
                  out, lse, dout, causal: bool = True, cu_seqlens=None,
                  scale: Optional[float] = None):
    """Backward of ``rank``'s share over the virtual ring.

    dq [b, L, h, d] is this rank's full query gradient.  dk_ring/dv_ring
    [N, b, L, h, d] hold the contributions of this rank's queries to every
    block's key/value gradient; summing them over all ranks gives the full
    gradients.  ``out``/``lse`` are the rank's FINAL forward results.
    """
    q_local = _f64(q_local)
    B, L, H, Dh = q_local.shape
    S = L * world
    qpos = layout_positions(layout, S, world, rank, cu_seqlens)
    dq = np.zeros_like(q_local)
    dk_ring = np.zeros(np.shape(k_ring), dtype=np.float64)
    dv_ring = np.zeros(np.shape(v_ring), dtype=np.float64)
    for src in ring_sources(world, rank):
        kpos = layout_positions(layout, S, world, src, cu_seqlens)
        a, b_, c = attention_backward(q_local, k_ring[src], v_ring[src], out, lse, dout,
                                      qpos, kpos, causal, cu_seqlens, scale)
        dq += a
        dk_ring[src] += b_
        dv_ring[src] += c
    return dq, dk_ring, dv_ring


# ---------------------------------------------------------------------------
# Helpers for tests: gathering a global tensor into the ring's block order
# ---------------------------------------------------------------------------

def to_ring(x_global, layout: str, world: int, cu_seqlens=None) -> np.ndarray:
    """[b, S, h, d] -> [N, b, S/N, h, d] by the oracle's own layout positions."""
    x_global = np.asarray(x_global)
    S = x_global.shape[1]
    return np.stack([x_global[:, layout_positions(layout, S, world, r, cu_seqlens)] for r in range(world)])

