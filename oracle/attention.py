"""Scaled dot-product attention by its plain definition, in fp64.

For every batch b, head h and query row i, with global positions
``q_pos0 + i`` for queries and ``k_pos0 + j`` for keys, and the visible set
J(i) (keys below ``valid_len``; for causal attention also j <= i):

    s_ij  = scale * sum_d Q[b,i,h,d] K[b,j,h,d]
    M_i   = max_{j in J(i)} s_ij
    l_i   = sum_{j in J(i)} exp(s_ij - M_i)
    O_i   = sum_{j in J(i)} exp(s_ij - M_i) V[b,j,h,:] / l_i
    LSE_i = M_i + ln l_i

This is the equation of §3.1 of the Ring Attention tutorial
(O = softmax(Q K^T / sqrt(d)) V, taken per (batch, head) over the sequence
with d the head dimension), stabilised by subtracting the row maximum as the
tutorial's §3.2 closing remark and §09 do.  The juejin post's reference code
(§二, §三) multiplies the last two axes of a [B, S, H, D] tensor, which would
attend across heads; the oracle reads it, as the tutorial's formula and the
Ulysses guideline's einsum over 'bshd,bthd' do, as attention over S per head.

A row with no visible key has O = 0, l = 0, M = LSE = -inf (never NaN).

Parity: pinned -- by the tutorial's printed 4 x 2 worked example (§04),
by torch's fp64 CPU scaled_dot_product_attention on full non-causal inputs,
by the prefix-mean closed form with equal keys (causal, global positions),
by constant-V and +1000-shift invariances, and by a pure-Python brute force
on tiny inputs (tests/test_oracle_pins.py).  ``gqa_expand`` (the K/V head a
query head reads under grouped-query attention) is pinned by the identity at
H_kv = H, by a per-head loop over the head map, and by the multi-query
invariances; ``packed_attention`` by a brute force with an explicit
same-sample mask and by the single-sample special case
(tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

from .schedule import visible_mask


def _f64(x) -> np.ndarray:
    """Exact fp64 copy of a numpy array or torch tensor (bf16 included)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale):
    """s[b,h,i,j] = scale * <q[b,i,h,:], k[b,j,h,:]> (fp64, no masking)."""
    q = _f64(q)
    k = _f64(k)
    out = np.empty((q.shape[0], q.shape[2], q.shape[1], k.shape[1]))
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            out[b, h] = scale * (q[b, :, h, :] @ k[b, :, h, :].T)
    return out


def attention(q, k, v, *, scale=None, causal=False, q_pos0=0, k_pos0=0,
              valid_len=None, rows=None, row_chunk=1024):
    """Attention of q [B,Sq,H,D] over k, v [B,Sk,H,D], in fp64.

    ``rows``: optional sorted array of query rows to compute (sampling for
    large shares); the outputs then have ``len(rows)`` on the row axis.
    Returns (o [B,R,H,D], lse [B,R,H], m [B,R,H], l [B,R,H]); m is the
    maximum of the scaled scores and l = sum exp(s - m), both natural base.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if valid_len is None:
        valid_len = np.iinfo(np.int64).max
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.zeros((B, R, H, v.shape[-1]))
    lse = np.full((B, R, H), -np.inf)
    m_out = np.full((B, R, H), -np.inf)
    l_out = np.zeros((B, R, H))
    k_pos = k_pos0 + np.arange(Sk)
    for c0 in range(0, R, row_chunk):
        rr = rows[c0:c0 + row_chunk]
        vis = visible_mask(q_pos0 + rr, k_pos, causal, valid_len)
        any_vis = vis.any(axis=1)
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, rr, h, :] @ k[b, :, h, :].T)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                m_safe = np.where(any_vis, m, 0.0)
                p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
                l = p.sum(axis=1)
                u = p @ v[b, :, h, :]
                l_safe = np.where(any_vis, l, 1.0)
                o[b, c0:c0 + len(rr), h, :] = np.where(any_vis[:, None],
                                                       u / l_safe[:, None], 0.0)
                m_out[b, c0:c0 + len(rr), h] = np.where(any_vis, m, -np.inf)
                l_out[b, c0:c0 + len(rr), h] = np.where(any_vis, l, 0.0)
                lse[b, c0:c0 + len(rr), h] = np.where(
                    any_vis, m + np.log(l_safe), -np.inf)
    return o, lse, m_out, l_out


def local_only_attention(q_r, k_r, v_r, *, scale=None, causal=False,
                         pos0=0, valid_len=None):
    """The negative control: a rank attending only to its own K/V shard.

    This is what the faulty library of the juejin post (§二 step 4, §三
    check [3]) returned; a correct ring output must differ from it.
    """
    o, _, _, _ = attention(q_r, k_r, v_r, scale=scale, causal=causal,
                           q_pos0=pos0, k_pos0=pos0, valid_len=valid_len)
    return o


def gqa_expand(x, H):
    """K or V [B, S, H_kv, D] seen by H query heads: query head h reads K/V
    head h // (H / H_kv) (grouped-query attention, named by the Ring
    Attention tutorial §3.5 and §6 as the case with fewer K/V heads than
    query heads).  Returns [B, S, H, D]; H_kv = H is the identity."""
    x = _f64(x)
    Hkv = x.shape[2]
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"{H} query heads are not a multiple of {Hkv} K/V heads")
    return x[:, :, np.arange(H) // (H // Hkv)]


def packed_attention(q, k, v, cu_seqlens, *, scale=None, causal=True, q_pos0=0, rows=None):
    """Attention over a packed sequence (B = 1): sample i holds global
    positions [cu_seqlens[i], cu_seqlens[i+1]) and a query attends only to
    keys of its own sample (the Ring Attention tutorial §6: packed sequences
    carry their boundaries and blocks never attend across samples).

    q: [1, Sq, H, D] at global positions q_pos0 + row; k, v: [1, S, H, D]
    from position 0.  Computed sample by sample with ``attention``: each
    sample is an independent sequence at its own global positions.  Rows
    outside every sample get o = 0, lse = -inf.  Returns (o, lse).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    _, Sq, H, D = q.shape
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((1, len(rows), H, v.shape[-1]))
    lse = np.full((1, len(rows), H), -np.inf)
    pos = q_pos0 + rows
    for s0, s1 in zip(cu_seqlens[:-1], cu_seqlens[1:]):
        sel = np.flatnonzero((pos >= s0) & (pos < s1))
        if len(sel) == 0:
            continue
        oi, li, _, _ = attention(q, k[:, s0:s1], v[:, s0:s1], scale=scale, causal=causal,
                                 q_pos0=q_pos0, k_pos0=s0, rows=rows[sel])
        o[:, sel] = oi
        lse[:, sel] = li
    return o, lse
