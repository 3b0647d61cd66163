"""Shard cover, padding, ring order and causal block classes (integer work).

Parity: pinned.  ``padded_len`` by the printed test of "Finalize guidelines for
Ulysses-based context-parallel attention" (§七: 3000 rejected, 3008 accepted,
3000 padded to 3008 for four ranks); ``shard_range`` by the cover invariants of the juejin post §三 (check [1])
and by the per-rank figures of the budget script in the Ring Attention
tutorial §04 (16384 local tokens, 8 rounds at L=131072, P=8);
``classify_block`` by brute force over ``visible_mask``; ``ring_sources`` by
the rule of the tutorial §3.3 and by the visited-block count of the causal
ring.  The zigzag helpers (tutorial §3.4's load-balanced sharding, read as:
2P chunks, rank r holding chunks r and 2P-1-r) are pinned by the cover of
the sequence, by the closed-form visible-pair count c (2P c + 1) per rank,
and by brute-force classes over ``visible_mask``.
"""
from __future__ import annotations

import numpy as np

SKIP, FULL, DIAG = 0, 1, 2


def padded_len(S: int, P: int, pad_multiple: int = 16) -> int:
    """Smallest multiple of P * pad_multiple that is >= S.

    The Ulysses guideline page (§六) pads the sequence to a multiple of
    cp_size * pad_multiple.  Its printed formula lost a '+' in extraction
    (read as the ceiling), and its own test (§七) rejects S = 3000 for four
    ranks and expects 3008 -- although 3000 = 4 * 750.  Those assertions hold
    together only if the unit is larger than P; reading pad_multiple as the
    per-rank granularity, 16 tokens (one key step of the matrix-core
    contraction) makes all of them true, and is the default here.
    """
    if P <= 0 or S < 0 or pad_multiple <= 0:
        raise ValueError("need P > 0, pad_multiple > 0 and S >= 0")
    unit = P * pad_multiple
    return -(-S // unit) * unit


def seq_divisible(S: int, P: int, pad_multiple: int = 16) -> bool:
    """The guideline's divisibility check (§六 validate_config, §七 test)."""
    return S % (P * pad_multiple) == 0


def shard_range(rank: int, P: int, S_padded: int):
    """Rank ``rank`` owns the contiguous rows [rank*S'/P, (rank+1)*S'/P).

    Contiguous, equal, non-overlapping shards in rank order (juejin post §三,
    shard-cover check; equal split once padded, guideline page §四).
    """
    if S_padded % P:
        raise ValueError(f"sequence length {S_padded} not divisible by P={P}; "
                         f"pad to {padded_len(S_padded, P, 1)}")
    if not 0 <= rank < P:
        raise ValueError("rank out of range")
    per = S_padded // P
    return rank * per, (rank + 1) * per


def ring_sources(P: int, rank: int):
    """Block visited at round t = 0..P-1: source (rank - t) mod P
    (Ring Attention tutorial §3.3)."""
    return [(rank - t) % P for t in range(P)]


def visible_mask(q_pos, k_pos, causal: bool, valid_len: int):
    """Boolean [len(q_pos), len(k_pos)]: may query i attend key j?

    A key is visible when it is a real key (global position < valid_len) and,
    for causal attention, not in the query's future on *global* positions
    (j <= i; tutorial §3.4, and §09 on global vs local indices).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)[:, None]
    k_pos = np.asarray(k_pos, dtype=np.int64)[None, :]
    vis = k_pos < valid_len
    if causal:
        vis = vis & (k_pos <= q_pos)
    return np.broadcast_to(vis, (q_pos.shape[0], k_pos.shape[1])).copy()


def classify_block(q0: int, q1: int, k0: int, k1: int, causal: bool,
                   valid_len: int) -> int:
    """Brute-force block class of query rows [q0,q1) against keys [k0,k1).

    Builds the whole element mask and reads the class off it: nothing
    visible -> SKIP, everything visible -> FULL, mixed -> DIAG (tutorial §3.4:
    a block wholly in the future is skipped, wholly in the past needs no
    mask, an overlapping one gets the triangular mask).
    """
    if q1 <= q0 or k1 <= k0:
        return SKIP
    m = visible_mask(np.arange(q0, q1), np.arange(k0, k1), causal, valid_len)
    if not m.any():
        return SKIP
    if m.all():
        return FULL
    return DIAG


def ring_schedule(P: int, rank: int, block_len: int, causal: bool,
                  valid_len: int):
    """(sources, classes) for every round of rank ``rank``'s ring.

    Sources follow the ring order; classes come from ``classify_block`` on
    the global ranges of the rank's query shard and the visited block.
    """
    q0, q1 = rank * block_len, (rank + 1) * block_len
    srcs = ring_sources(P, rank)
    cls = [classify_block(q0, q1, j * block_len, (j + 1) * block_len, causal,
                          valid_len) for j in srcs]
    return srcs, cls


# ---------------------------------------------------------------- zigzag
# Tutorial §3.4: with contiguous shards the causal ring gives rank r the
# work of r + 1/2 blocks; implementations rebalance it by letting every rank
# hold both early and late positions.  Reading adopted (the page names the
# idea only): cut the sequence into 2P equal chunks; rank r holds chunk r
# followed by chunk 2P-1-r.

def zigzag_chunks(P: int, rank: int):
    """The two chunk indices of rank ``rank``'s share, in share order."""
    return rank, 2 * P - 1 - rank


def zigzag_positions(P: int, rank: int, chunk_len: int) -> np.ndarray:
    """Global positions of the rows of rank ``rank``'s share, in share order."""
    a, b = zigzag_chunks(P, rank)
    return np.concatenate([a * chunk_len + np.arange(chunk_len),
                           b * chunk_len + np.arange(chunk_len)])


def zigzag_schedule(P: int, rank: int, chunk_len: int, causal: bool,
                    valid_len: int):
    """(sources, classes): round t visits the share of rank (rank - t) mod P
    (tutorial §3.3); classes[t] = (class of its first chunk, class of its
    second chunk) against the rank's query positions, by brute force."""
    q_pos = zigzag_positions(P, rank, chunk_len)
    srcs = ring_sources(P, rank)
    cls = []
    for j in srcs:
        pair = []
        for kc in zigzag_chunks(P, j):
            m = visible_mask(q_pos, kc * chunk_len + np.arange(chunk_len), causal,
                             valid_len)
            pair.append(SKIP if not m.any() else (FULL if m.all() else DIAG))
        cls.append(tuple(pair))
    return srcs, cls


def visible_pairs(q_pos, P: int, S: int, causal: bool, valid_len: int) -> int:
    """Number of visible (query, key) pairs of the given query positions over
    keys 0 .. S-1 (brute force)."""
    return int(visible_mask(q_pos, np.arange(S), causal, valid_len).sum())
