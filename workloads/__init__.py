"""Seeded synthetic inputs for ring-order block attention and the Ulysses transposes.

This module holds the workload table and the input generators only.  It does
no attention arithmetic, so both the HIP path (through the Python binding) and
the fp64 oracle can be fed from it without sharing any of the method's code.

Recipe (the verification scripts of "How I found a sequence-parallel attention
library that never communicated" (juejin, section 3) draw Q, K and V from one
seeded generator, in that order, with shape [B, S, H, D]):

* ``torch.Generator(device).manual_seed(seed)``; ``torch.randn`` in fp32 over
  the *real* global shape ``[B, S, H, D]``, drawn in the order q, k, v;
* optional outlier rows (see ``Workload.outlier_k_scale``) are multiplied in
  fp32 before any cast;
* bf16 workloads are then rounded to bf16 (round-to-nearest-even, torch's
  ``.to(torch.bfloat16)``);
* when the global length is padded to a multiple of P, zero rows are appended
  at the end of the sequence axis *after* generation, so the real rows are the
  same with or without padding.

Large workloads may be generated on the GPU (``device="cuda"``): the values
then come from torch's device generator rather than the CPU one, but the
oracle always receives exact host copies of the very tensors the GPU sees.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    ``S`` is the real global sequence length; ``P`` the sequence-parallel
    degree.  ``ranks`` lists the ranks whose share is computed.
    """

    name: str
    dtype: str            # "fp32" or "bf16"
    B: int
    S: int
    H: int
    D: int
    P: int
    causal: bool
    ranks: tuple
    ulysses: bool = False
    # C5: multiply one K row per (b, h) by this factor (None = no outliers)
    outlier_k_scale: Optional[float] = None
    seed: int = 0
    note: str = ""
    # zigzag sharding: 2P chunks, rank r holds chunks r and 2P-1-r
    zigzag: bool = False

    pad_multiple: int = 16

    @property
    def S_padded(self) -> int:
        """Global length padded to a multiple of P * pad_multiple."""
        unit = self.P * self.pad_multiple
        return ((self.S + unit - 1) // unit) * unit

    @property
    def block_len(self) -> int:
        return self.S_padded // self.P

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


# The five configurations of the ring / Ulysses workload family.
TINY_FP32 = Workload(
    name="tiny_fp32_ring", dtype="fp32", B=1, S=256, H=2, D=64, P=2,
    causal=False, ranks=(0, 1),
    note="tiny fp32 ring attention; every rank's share")
DIT_SHARD = Workload(
    name="dit_latent_shard", dtype="bf16", B=1, S=4096, H=24, D=128, P=4,
    causal=False, ranks=(0, 1, 2, 3),
    note="diffusion-transformer latent sequence (64x64 patches), 4-way ring")
ULYSSES = Workload(
    name="ulysses_layout", dtype="bf16", B=1, S=16384, H=32, D=128, P=8,
    causal=False, ranks=tuple(range(8)), ulysses=True,
    note="seq-shard -> head-shard, full attention on H/P heads, inverse")
LONG_CAUSAL = Workload(
    name="long_context_causal_rank3", dtype="bf16", B=1, S=131072, H=64,
    D=128, P=8, causal=True, ranks=(3,),
    note="L=131072, hidden 8192 = 64 x 128, P=8, rank 3's share")
PADDED_CAUSAL = Workload(
    name="padded_causal", dtype="bf16", B=2, S=3000, H=16, D=64, P=4,
    causal=True, ranks=(0, 1, 2, 3), outlier_k_scale=8.0,
    note="S=3000 padded to 3008, one K row per (b,h) scaled x8")

# Zigzag (load-balanced) sharding of the same shapes: chunks of a multiple
# of 64 rows, so the padding unit is P * 128.
LONG_ZIGZAG = Workload(
    name="long_context_causal_zigzag", dtype="bf16", B=1, S=131072, H=64,
    D=128, P=8, causal=True, ranks=(0, 7), zigzag=True, pad_multiple=128,
    note="L=131072, P=8, zigzag shares (chunks r and 15-r of 8192 rows)")
PADDED_ZIGZAG = Workload(
    name="padded_causal_zigzag", dtype="bf16", B=2, S=3000, H=16, D=64, P=4,
    causal=True, ranks=(0, 1, 2, 3), outlier_k_scale=8.0, zigzag=True,
    pad_multiple=128, note="S=3000 padded to 3072, zigzag chunks of 384")

CONFIGS = (TINY_FP32, DIT_SHARD, ULYSSES, LONG_CAUSAL, PADDED_CAUSAL)
ZIGZAG_CONFIGS = (LONG_ZIGZAG, PADDED_ZIGZAG)
BY_NAME = {c.name: c for c in CONFIGS + ZIGZAG_CONFIGS}


def outlier_token(b: int, h: int, block_len: int) -> int:
    """Token index of the scaled K row for (b, h): inside block 0, spread over
    heads and batches so that different rows carry the outlier."""
    return (47 * h + 13 * b) % block_len


def make_qkv(w: Workload, device: str = "cpu", seed: Optional[int] = None):
    """Return (q, k, v) of shape [B, S_padded, H, D] in the workload dtype.

    Rows ``S .. S_padded-1`` are zero padding.  The tensors live on
    ``device``; generation happens there too.
    """
    seed = w.seed if seed is None else seed
    g = torch.Generator(device=device).manual_seed(seed)
    shape = (w.B, w.S, w.H, w.D)
    q = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.outlier_k_scale is not None:
        for b in range(w.B):
            for h in range(w.H):
                k[b, outlier_token(b, h, w.block_len), h, :] *= w.outlier_k_scale
    out = []
    for x in (q, k, v):
        x = x.to(w.torch_dtype)
        if w.S_padded != w.S:
            pad = torch.zeros((w.B, w.S_padded - w.S, w.H, w.D),
                              dtype=x.dtype, device=device)
            x = torch.cat([x, pad], dim=1)
        out.append(x.contiguous())
    return tuple(out)


def random_tensor(shape, dtype=torch.bfloat16, seed: int = 0, device="cpu"):
    """N(0,1) tensor of ``shape`` cast to ``dtype`` (seeded)."""
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(shape, generator=g, device=device,
                       dtype=torch.float32).to(dtype).contiguous()


def random_bits16(shape, seed: int = 0, device="cpu"):
    """Uniform random 16-bit patterns (as int16), including NaN payloads and
    negative zero; for bit-exactness tests of the layout permutations."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randint(-32768, 32768, shape, generator=g, device=device,
                      dtype=torch.int32).to(torch.int16)
    flat = x.view(-1)
    if flat.numel() >= 4:
        flat[0] = -32768          # 0x8000: bf16 negative zero
        flat[1] = 0x7FC1          # bf16 quiet NaN with payload
        flat[2] = -129            # 0xFF7F: bf16 -max finite
        flat[3] = 0x7F80          # bf16 +inf
    return x.contiguous()
