"""Ulysses sequence-shard <-> head-shard transposes as index maps.

The Ring Attention tutorial §3.5: the Ulysses all-to-all turns the
sequence-sharded layout [B, L/P, H, D_h] into the head-sharded layout
[B, L, H/P, D_h] (each rank then holds the whole sequence for H/P heads) and
a second all-to-all turns the output back.  On one GPU the P per-rank
tensors are stacked rank-major; with Sl = L/P and Hl = H/P, head group r is
the contiguous heads [r*Hl, (r+1)*Hl) and sequence shard j the rows
[j*Sl, (j+1)*Sl):

    head[r, b, j*Sl + s, h', d] = seq[j, b, s, r*Hl + h', d]
    seq[j, b, s, r*Hl + h', d]  = head[r, b, j*Sl + s, h', d]

These are pure data movement: the maps copy stored bit patterns and never
interpret them as numbers.

Parity: pinned -- the slice form agrees with the element-by-element loops on
small shapes, the two maps invert each other, and rank r's head-shard tensor
equals the rows of the re-assembled global sequence restricted to head group
r (the tutorial's description of what each rank sees after the all-to-all).
"""
from __future__ import annotations

import numpy as np


def _np(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


def seq2head(x_seq):
    """[P, B, Sl, H, D] -> [P, B, P*Sl, H/P, D] by block slices."""
    x = _np(x_seq)
    P, B, Sl, H, D = x.shape
    if H % P:
        raise ValueError(f"H={H} not divisible by P={P}")
    Hl = H // P
    out = np.empty((P, B, P * Sl, Hl, D), dtype=x.dtype)
    for r in range(P):
        for j in range(P):
            out[r, :, j * Sl:(j + 1) * Sl] = x[j, :, :, r * Hl:(r + 1) * Hl]
    return out


def head2seq(x_head):
    """[P, B, S, Hl, D] -> [P, B, S/P, P*Hl, D] by block slices."""
    x = _np(x_head)
    P, B, S, Hl, D = x.shape
    if S % P:
        raise ValueError(f"S={S} not divisible by P={P}")
    Sl = S // P
    out = np.empty((P, B, Sl, P * Hl, D), dtype=x.dtype)
    for j in range(P):
        for r in range(P):
            out[j, :, :, r * Hl:(r + 1) * Hl] = x[r, :, j * Sl:(j + 1) * Sl]
    return out


def seq2head_loops(x_seq):
    """Element-by-element form of ``seq2head`` (tiny shapes only)."""
    x = _np(x_seq)
    P, B, Sl, H, D = x.shape
    Hl = H // P
    out = np.empty((P, B, P * Sl, Hl, D), dtype=x.dtype)
    for r in range(P):
        for b in range(B):
            for j in range(P):
                for s in range(Sl):
                    for hh in range(Hl):
                        for d in range(D):
                            out[r, b, j * Sl + s, hh, d] = x[j, b, s, r * Hl + hh, d]
    return out


def head2seq_loops(x_head):
    """Element-by-element form of ``head2seq`` (tiny shapes only)."""
    x = _np(x_head)
    P, B, S, Hl, D = x.shape
    Sl = S // P
    out = np.empty((P, B, Sl, P * Hl, D), dtype=x.dtype)
    for j in range(P):
        for b in range(B):
            for s in range(Sl):
                for r in range(P):
                    for hh in range(Hl):
                        for d in range(D):
                            out[j, b, s, r * Hl + hh, d] = x[r, b, j * Sl + s, hh, d]
    return out
