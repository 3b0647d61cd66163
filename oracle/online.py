"""The ring: online-softmax recurrence over K/V blocks, and the LSE combine.

``ring_attention_rank`` follows §3.2-§3.4 of the Ring Attention tutorial step
by step, in its notation: per query row keep the running maximum m, the
denominator l and the unnormalised weighted sum u; visit the blocks in ring
order (source (r - t) mod P at round t); for each visited block with scores s
    m_b      = max_j s_j
    m_{t+1}  = max(m_t, m_b)
    alpha    = exp(m_t - m_{t+1})          (0 while m_t is still -inf)
    l_{t+1}  = alpha l_t + sum_j exp(s_j - m_{t+1})
    u_{t+1}  = alpha u_t + sum_j exp(s_j - m_{t+1}) v_j
and finish with o = u_T / l_T.  A block whose element mask is empty for the
whole query shard is skipped (future block); a block that is wholly visible
needs no mask; the rest get the element mask on global positions.

``lse_combine`` is the pairwise merge of the juejin post (§四, §五):
lse = logaddexp(lse1, lse2), o = o1 exp(lse1 - lse) + o2 exp(lse2 - lse),
extended so that two empty partials (lse = -inf) merge to (0, -inf).

``composable_ring_rank`` is the same ring done the post's way: per-round
partial attention (o, lse) of one block, folded in with ``lse_combine``.

``zigzag_ring_rank`` runs the same recurrence over zigzag shares (tutorial
§3.4's load balancing; see ``schedule.zigzag_positions``): the rank's
queries sit at two ranges of global positions and round t brings the two
chunks of rank (r - t) mod P's share, each at its own positions.

Parity: pinned -- all three agree with the plain definition in ``attention`` to
<= 1e-12 for 1, 2, 4, 8 and 16 chunks and block sizes 1, 2, 4 (the post
reports ~1e-16 for its pure-Python check, the tutorial max_abs_diff = 0 for its
worked example), survive a +1000 shift of all scores (tutorial §09), and the
recurrence reproduces the tutorial's printed ring[0] of the 4 x 2 example.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attention
from .schedule import SKIP, ring_sources, visible_mask, zigzag_chunks, zigzag_positions


def ring_attention_rank(q_r, k_blocks, v_blocks, rank, *, scale=None,
                        causal=False, valid_len=None, rows=None,
                        return_trace=False):
    """Rank ``rank``'s output by the (m, l, u) recurrence in ring order.

    q_r: [B, Sb, H, D] (rank's query shard, global rows rank*Sb ...);
    k_blocks / v_blocks: P arrays [B, Sb, H, D], block j holding global rows
    j*Sb ... (j+1)*Sb - 1.  Returns (o, lse) and, with ``return_trace``, the
    list of (round, source, visited) triples.
    """
    P = len(k_blocks)
    q = _f64(q_r)
    B, Sb, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = P * Sb
    rows = np.arange(Sb) if rows is None else np.asarray(rows, dtype=np.int64)
    q = q[:, rows]
    q_pos = rank * Sb + rows
    R = rows.shape[0]
    m = np.full((B, R, H), -np.inf)
    l = np.zeros((B, R, H))
    u = np.zeros((B, R, H, _f64(v_blocks[0]).shape[-1]))
    trace = []
    for t, j in enumerate(ring_sources(P, rank)):
        k_pos = j * Sb + np.arange(Sb)
        vis = visible_mask(q_pos, k_pos, causal, valid_len)
        # the block as a whole: skip only when no (query, key) pair is visible
        # over the whole shard -- never merely because the ring is causal
        shard_vis = visible_mask(rank * Sb + np.arange(Sb), k_pos, causal,
                                 valid_len)
        if not shard_vis.any():
            trace.append((t, j, False))
            continue
        trace.append((t, j, True))
        kj = _f64(k_blocks[j])
        vj = _f64(v_blocks[j])
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, :, h, :] @ kj[b, :, h, :].T)
                s = np.where(vis, s, -np.inf)
                m_b = s.max(axis=1)
                m_old = m[b, :, h]
                m_new = np.maximum(m_old, m_b)
                finite = np.isfinite(m_new)
                m_ref = np.where(finite, m_new, 0.0)
                alpha = np.where(np.isfinite(m_old), np.exp(m_old - m_ref), 0.0)
                p = np.where(vis, np.exp(s - m_ref[:, None]), 0.0)
                l[b, :, h] = alpha * l[b, :, h] + p.sum(axis=1)
                u[b, :, h, :] = alpha[:, None] * u[b, :, h, :] + p @ vj[b, :, h, :]
                m[b, :, h] = m_new
    seen = l > 0
    o = np.where(seen[..., None], u / np.where(seen, l, 1.0)[..., None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    if return_trace:
        return o, lse, trace
    return o, lse


def lse_combine(o1, lse1, o2, lse2):
    """Merge two normalised partial outputs by their log-sum-exp weights."""
    o1 = _f64(o1)
    o2 = _f64(o2)
    lse1 = _f64(lse1)
    lse2 = _f64(lse2)
    lse = np.logaddexp(lse1, lse2)
    finite = np.isfinite(lse)
    lse_ref = np.where(finite, lse, 0.0)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - lse_ref), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - lse_ref), 0.0)
    return o1 * w1[..., None] + o2 * w2[..., None], lse


def composable_ring_rank(q_r, k_blocks, v_blocks, rank, *, scale=None,
                         causal=False, valid_len=None):
    """Ring output built from per-round partials and ``lse_combine``.

    Every round's partial is the plain attention of the rank's queries over
    one block (global positions), including an empty partial for a future
    block; merging an empty partial changes nothing.
    """
    P = len(k_blocks)
    q = _f64(q_r)
    Sb = q.shape[1]
    if valid_len is None:
        valid_len = P * Sb
    o = lse = None
    for j in ring_sources(P, rank):
        oj, lj, _, _ = attention(q, k_blocks[j], v_blocks[j], scale=scale,
                                 causal=causal, q_pos0=rank * Sb,
                                 k_pos0=j * Sb, valid_len=valid_len)
        if o is None:
            o, lse = oj, lj
        else:
            o, lse = lse_combine(o, lse, oj, lj)
    return o, lse


def chunked_attention(q, k, v, n_chunks, *, scale=None, causal=False):
    """Whole-sequence attention with K/V cut into ``n_chunks`` equal chunks,
    visited in order and merged by ``lse_combine`` (the juejin post's §五
    single-process simulation of a ring)."""
    k = _f64(k)
    v = _f64(v)
    Sk = k.shape[1]
    if Sk % n_chunks:
        raise ValueError("chunk count must divide the key length")
    per = Sk // n_chunks
    o = lse = None
    for c in range(n_chunks):
        sl = slice(c * per, (c + 1) * per)
        oc, lc, _, _ = attention(q, k[:, sl], v[:, sl], scale=scale,
                                 causal=causal, q_pos0=0, k_pos0=c * per)
        if o is None:
            o, lse = oc, lc
        else:
            o, lse = lse_combine(o, lse, oc, lc)
    return o, lse


__all__ = ["ring_attention_rank", "lse_combine", "composable_ring_rank",
           "chunked_attention", "SKIP"]


def zigzag_ring_rank(q_share, k_shares, v_shares, rank, *, scale=None,
                     causal=True, valid_len=None):
    """Rank ``rank``'s output over zigzag shares by the (m, l, u) recurrence.

    q_share and every share: [B, 2c, H, D], chunk r then chunk 2P-1-r of the
    sequence (r the owner).  Round t visits share (rank - t) mod P, first
    chunk then second chunk, each at its global positions; a chunk with no
    visible pair for any query of the share is skipped.  Returns (o, lse).
    """
    P = len(k_shares)
    q = _f64(q_share)
    B, Sr, H, D = q.shape
    c = Sr // 2
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = P * Sr
    q_pos = zigzag_positions(P, rank, c)
    m = np.full((B, Sr, H), -np.inf)
    l = np.zeros((B, Sr, H))
    u = np.zeros((B, Sr, H, D))
    for j in ring_sources(P, rank):
        kj = _f64(k_shares[j])
        vj = _f64(v_shares[j])
        for half, kc in enumerate(zigzag_chunks(P, j)):
            k_pos = kc * c + np.arange(c)
            vis = visible_mask(q_pos, k_pos, causal, valid_len)
            if not vis.any():
                continue
            kk = kj[:, half * c:(half + 1) * c]
            vv = vj[:, half * c:(half + 1) * c]
            for b in range(B):
                for h in range(H):
                    s = scale * (q[b, :, h, :] @ kk[b, :, h, :].T)
                    s = np.where(vis, s, -np.inf)
                    m_old = m[b, :, h]
                    m_new = np.maximum(m_old, s.max(axis=1))
                    m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.where(np.isfinite(m_old), np.exp(m_old - m_ref), 0.0)
                    p = np.where(vis, np.exp(s - m_ref[:, None]), 0.0)
                    l[b, :, h] = alpha * l[b, :, h] + p.sum(axis=1)
                    u[b, :, h, :] = alpha[:, None] * u[b, :, h, :] + p @ vv[b, :, h, :]
                    m[b, :, h] = m_new
    seen = l > 0
    o = np.where(seen[..., None], u / np.where(seen, l, 1.0)[..., None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return o, lse
