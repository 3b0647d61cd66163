"""Gradients of attention and the ring backward, in fp64.

``attention_grad`` is the plain definition: the gradients of the scalar
L = sum(dO * O) for O = attention(Q, K, V) of ``attention.py``, by the chain
rule through the row softmax.  Per (batch, head), with P the softmax of the
masked scaled scores and D_i = sum_d dO_id O_id:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D)            (D broadcast along the keys)
    dQ = scale * dS K
    dK = scale * dS^T Q

A row with no visible key has P = 0 and contributes nothing.

``ring_attention_bwd_rank`` follows the Ring Attention tutorial's account of
the backward (§3.3 closing paragraph, §6.2): rank r keeps Q_r, dO_r and the
forward's per-row statistics; when the K/V block of source j arrives (ring
order (r - t) mod P, future blocks skipped when causal) it recomputes the
local scores and probabilities from the saved log-sum-exp,
P_j = exp(S_j - lse_r), adds the block's term to dQ_r and produces the parts
dK_j, dV_j that belong to rank j -- to be summed over every query shard and
returned to the owner.  The function returns dQ_r and those parts.

Parity: pinned -- ``attention_grad`` by central finite differences of L on
tiny inputs (causal, padded, non-causal), by torch's fp64 autograd of
scaled_dot_product_attention, and by the invariants sum_j dK_j = 0 and
sum_j dV_j = sum_i dO_i (rows with a visible key); ``ring_attention_bwd_rank``
by the ring decomposition (the owners' sums over all ranks equal the
full-sequence gradients to fp64 rounding) and by two planted mistakes (parts
returned to the wrong owner; probabilities from a block-local instead of the
global log-sum-exp) that must fail; ``attention_grad_sampled`` by equality
with the selected rows of ``attention_grad`` (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, attention
from .schedule import ring_sources, visible_mask


def _discard_pad_rows(do, q_pos, valid_len):
    """dO with the rows of padding queries (global position >= valid_len)
    set to zero: padding queries are computed but discarded (the
    Ulysses guidelines pad the sequence and drop the pad rows of the
    output), so they are not part of the loss and none of their terms
    reaches any gradient."""
    real = np.asarray(q_pos, dtype=np.int64) < valid_len
    return np.where(real[None, :, None, None], do, 0.0)


def attention_grad(q, k, v, do, *, scale=None, causal=False, q_pos0=0, k_pos0=0,
                   valid_len=None):
    """(dq, dk, dv) of L = sum(do * attention(q, k, v)) over the real query
    rows (position < valid_len), all [B, S, H, D] fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = np.iinfo(np.int64).max
    do = _discard_pad_rows(do, q_pos0 + np.arange(Sq), valid_len)
    vis = visible_mask(q_pos0 + np.arange(Sq), k_pos0 + np.arange(Sk), causal, valid_len)
    any_vis = vis.any(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            s = np.where(vis, scale * (q[b, :, h] @ k[b, :, h].T), -np.inf)
            m = np.where(any_vis, s.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            den = np.where(any_vis, e.sum(axis=1), 1.0)
            p = e / den[:, None]
            o = p @ v[b, :, h]
            dsum = (do[b, :, h] * o).sum(axis=1)
            dp = do[b, :, h] @ v[b, :, h].T
            ds = p * (dp - dsum[:, None])
            dv[b, :, h] = p.T @ do[b, :, h]
            dq[b, :, h] = scale * (ds @ k[b, :, h])
            dk[b, :, h] = scale * (ds.T @ q[b, :, h])
    return dq, dk, dv


def ring_attention_bwd_rank(q_r, k_blocks, v_blocks, do_r, rank, *, o_r=None, lse_r=None,
                            scale=None, causal=False, valid_len=None, lse_block_local=False):
    """Rank ``rank``'s share of the ring backward.

    q_r, do_r: [B, Sb, H, D] (global rows rank*Sb ...); k_blocks / v_blocks:
    P arrays [B, Sb, H, D].  o_r / lse_r: the forward's output and natural
    log-sum-exp of the rank's rows (computed here when not given).  Returns
    (dq_r, dk_parts, dv_parts): dk_parts[j] / dv_parts[j] are the parts that
    belong to block j's owner (zeros for a block the rank skips).
    ``lse_block_local`` plants a mistake for the tests: probabilities
    normalised within each block instead of by the global log-sum-exp.
    """
    P = len(k_blocks)
    q = _f64(q_r)
    do = _f64(do_r)
    B, Sb, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = P * Sb
    if o_r is None or lse_r is None:
        kk = np.concatenate([_f64(x) for x in k_blocks], axis=1)
        vv = np.concatenate([_f64(x) for x in v_blocks], axis=1)
        o_f, lse_f, _, _ = attention(q, kk, vv, scale=scale, causal=causal, q_pos0=rank * Sb,
                                     k_pos0=0, valid_len=valid_len)
        o_r = o_f if o_r is None else o_r
        lse_r = lse_f if lse_r is None else lse_r
    o = _f64(o_r)
    lse = _f64(lse_r)
    q_pos = rank * Sb + np.arange(Sb)
    do = _discard_pad_rows(do, q_pos, valid_len)
    dsum = (do * o).sum(axis=3)                       # [B, Sb, H]
    dq = np.zeros_like(q)
    dk_parts = [np.zeros_like(q) for _ in range(P)]
    dv_parts = [np.zeros_like(q) for _ in range(P)]
    for j in ring_sources(P, rank):
        vis = visible_mask(q_pos, j * Sb + np.arange(Sb), causal, valid_len)
        if not vis.any():
            continue
        kj, vj = _f64(k_blocks[j]), _f64(v_blocks[j])
        for b in range(B):
            for h in range(H):
                s = np.where(vis, scale * (q[b, :, h] @ kj[b, :, h].T), -np.inf)
                if lse_block_local:
                    any_vis = vis.any(axis=1)
                    m = np.where(any_vis, s.max(axis=1), 0.0)
                    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
                    p = e / np.where(any_vis, e.sum(axis=1), 1.0)[:, None]
                else:
                    ref = np.where(np.isfinite(lse[b, :, h]), lse[b, :, h], 0.0)
                    p = np.where(vis, np.exp(s - ref[:, None]), 0.0)
                dp = do[b, :, h] @ vj[b, :, h].T
                ds = p * (dp - dsum[b, :, h][:, None])
                dq[b, :, h] += scale * (ds @ kj[b, :, h])
                dk_parts[j][b, :, h] += scale * (ds.T @ q[b, :, h])
                dv_parts[j][b, :, h] += p.T @ do[b, :, h]
    return dq, dk_parts, dv_parts


def attention_grad_sampled(q, k, v, do, o, lse, *, q_rows, k_rows, scale=None, causal=False,
                           q_pos0=0, k_pos0=0, valid_len=None):
    """Selected rows of (dq, dk, dv) from the saved forward statistics.

    Same gradients as ``attention_grad`` (P = exp(s - lse) over the visible
    pairs, D = rowsum(dO * O)), evaluated only for the query rows ``q_rows``
    (dq: each needs its scores against every key) and the key rows
    ``k_rows`` (dk, dv: each needs its scores against every query), so that
    a long share can be checked on a sample.  Returns (dq [B, |q_rows|, H, D],
    dk [B, |k_rows|, H, D], dv [B, |k_rows|, H, D]).
    """
    q, k, v, do, o, lse = (_f64(x) for x in (q, k, v, do, o, lse))
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = np.iinfo(np.int64).max
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    do = _discard_pad_rows(do, q_pos0 + np.arange(Sq), valid_len)
    dsum = (do * o).sum(axis=3)                                   # [B, Sq, H]
    lse_ref = np.where(np.isfinite(lse), lse, np.inf)            # no key seen: P = 0
    dq = np.zeros((B, len(q_rows), H, D))
    dk = np.zeros((B, len(k_rows), H, D))
    dv = np.zeros((B, len(k_rows), H, D))
    vis_q = visible_mask(q_pos0 + q_rows, k_pos0 + np.arange(Sk), causal, valid_len)
    vis_k = visible_mask(q_pos0 + np.arange(Sq), k_pos0 + k_rows, causal, valid_len)
    for b in range(B):
        for h in range(H):
            # rows: scores of the sampled queries against all keys
            s = scale * (q[b, q_rows, h] @ k[b, :, h].T)
            p = np.where(vis_q, np.exp(s - lse_ref[b, q_rows, h][:, None]), 0.0)
            ds = p * (do[b, q_rows, h] @ v[b, :, h].T - dsum[b, q_rows, h][:, None])
            dq[b, :, h] = scale * (ds @ k[b, :, h])
            # columns: scores of all queries against the sampled keys
            s = scale * (q[b, :, h] @ k[b, k_rows, h].T)
            p = np.where(vis_k, np.exp(s - lse_ref[b, :, h][:, None]), 0.0)
            ds = p * (do[b, :, h] @ v[b, k_rows, h].T - dsum[b, :, h][:, None])
            dk[b, :, h] = scale * (ds.T @ q[b, :, h])
            dv[b, :, h] = p.T @ do[b, :, h]
    return dq, dk, dv
