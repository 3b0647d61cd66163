"""The C ABI on the host: the library loads, exports every declared symbol,
and its host-side logic (padding, shard cover, ring order, block classes)
agrees with the oracle's brute force.  No GPU and no compute calls."""
import os
import re

import numpy as np
import pytest

import oracle
from oracle import schedule as sch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")

ra = pytest.importorskip("ring_ulysses_sequence_amd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ra.LIB_PATH):
        pytest.fail("libringattn.so is not built (run __graft_entry__.build())")
    return ra.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(ra.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    # the symbols are plain C (unmangled) exports of the shared object
    out = os.popen(f"nm -D --defined-only {ra.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_abi_version(lib):
    assert ra.abi_version() == 1


def test_kernel_option(lib):
    assert ra.get_attn_kernel() == ra.RA_KERNEL_AUTO
    for c in (ra.RA_KERNEL_BR128, ra.RA_KERNEL_BR256, ra.RA_KERNEL_W64, ra.RA_KERNEL_WS,
              ra.RA_KERNEL_PP,
              ra.RA_KERNEL_AUTO):
        ra.set_attn_kernel(c)
        assert ra.get_attn_kernel() == c
    with pytest.raises(RuntimeError):
        ra.set_attn_kernel(7)
    assert lib.ra_set_option(99, 0) == 4


def test_padded_len_matches_oracle(lib):
    for S in [0, 1, 15, 16, 3000, 3008, 4096, 131072, 131073]:
        for P in [1, 2, 3, 4, 8]:
            for m in [1, 16]:
                assert ra.padded_len(S, P, m) == sch.padded_len(S, P, m)
    assert ra.padded_len(3000, 4) == 3008
    with pytest.raises(ValueError):
        ra.padded_len(-1, 4)
    with pytest.raises(ValueError):
        ra.padded_len(10, 0)


def test_shard_range_matches_oracle_and_errors(lib):
    for S, P in [(3008, 4), (131072, 8), (64, 2), (12, 3)]:
        for r in range(P):
            assert ra.shard_range(S, P, r) == sch.shard_range(r, P, S)
    with pytest.raises(ValueError, match="3008"):
        ra.shard_range(3002, 4, 0)       # message names the padded length
    with pytest.raises(RuntimeError):
        ra.shard_range(64, 2, 2)          # rank out of range


def test_ring_schedule_matches_oracle(lib):
    for P in range(1, 9):
        for r in range(P):
            for causal in (False, True):
                for bl, vl in [(5, 5 * P), (16, 16 * P - 7), (752, 3000)]:
                    if vl <= 0:
                        continue
                    got = ra.ring_schedule(P, r, bl, causal, vl)
                    exp = sch.ring_schedule(P, r, bl, causal, vl)
                    assert got == (list(exp[0]), list(exp[1])), (P, r, causal, bl, vl)
    assert ra.ring_schedule(8, 3, 16384, True) == (
        [3, 2, 1, 0, 7, 6, 5, 4], [ra.RA_DIAG, ra.RA_FULL, ra.RA_FULL, ra.RA_FULL,
                                   ra.RA_SKIP, ra.RA_SKIP, ra.RA_SKIP, ra.RA_SKIP])
    with pytest.raises(RuntimeError):
        ra.ring_schedule(4, 4, 16, True)


def test_zigzag_schedule_matches_oracle(lib):
    """The library's zigzag ring (sources and chunk classes) equals the
    oracle's brute force over the share's positions, causal or not, with
    and without padding."""
    for P in (1, 2, 3, 4, 8):
        for c in (1, 3, 64):
            S = 2 * P * c
            for causal in (False, True):
                for valid in (S, S - 1, S - c - 1, c):
                    if valid <= 0:
                        continue
                    for r in range(P):
                        got = ra.zigzag_schedule(P, r, c, causal, valid)
                        want = sch.zigzag_schedule(P, r, c, causal, valid)
                        assert got[0] == want[0]
                        assert got[1] == [tuple(x) for x in want[1]], (P, c, causal, valid, r)


def test_zigzag_padded_len(lib):
    """Multiples of 2P * 64: the long-context share needs no padding, 3000
    tokens on four ranks pad to 3072; bad arguments are refused."""
    assert ra.zigzag_padded_len(131072, 8) == 131072
    assert ra.zigzag_padded_len(3000, 4) == 3072
    assert ra.zigzag_padded_len(0, 4) == 0
    with pytest.raises(ValueError):
        ra.zigzag_padded_len(10, 0)


def test_split_hint(lib):
    """Slices only while the grid of 128-row workgroups is under the chip's
    512 slots, a divisor of the visited blocks that minimises rounds x
    blocks per slice (+0.15 block per slice for the merge); -1 on bad
    sizes."""
    def model(base, vis):
        if vis <= 1 or base >= 512:
            return 1
        cost = {ns: 20 * -(-base * ns // 512) * (vis // ns) + 3 * ns
                for ns in range(1, vis + 1) if vis % ns == 0}
        return min(cost, key=lambda ns: (cost[ns], ns))
    # DiT shard: 24 heads x 8 row tiles = 192 workgroups, 4 blocks visited:
    # two slices (one round of 384) beat four (two rounds of 768)
    assert ra.ring_split_hint(1, 1024, 24, 4, 0) == 2 == model(192, 4)
    # causal rank 1 visits 2 blocks; rank 0 only its own
    assert ra.ring_split_hint(1, 1024, 24, 4, 1, causal=True) == 2
    assert ra.ring_split_hint(1, 1024, 24, 4, 0, causal=True) == 1
    # the long-context share fills the chip
    assert ra.ring_split_hint(1, 16384, 64, 8, 3, causal=True) == 1
    for B, Sb, H, P in [(1, 128 * 75, 4, 8), (2, 512, 4, 4), (1, 2048, 2, 6), (1, 640, 9, 3)]:
        base = B * H * -(-Sb // 128)
        assert ra.ring_split_hint(B, Sb, H, P, 0) == model(base, P), (B, Sb, H, P)
    with pytest.raises(ValueError):
        ra.ring_split_hint(1, 16, 1, 0, 0)


def test_classify_block_matches_brute_force(lib):
    rng = np.random.default_rng(11)
    for _ in range(3000):
        q0, k0 = (int(x) for x in rng.integers(0, 50, 2))
        q1 = q0 + int(rng.integers(0, 14))
        k1 = k0 + int(rng.integers(0, 14))
        vl = int(rng.integers(0, 70))
        causal = bool(rng.integers(0, 2))
        assert ra.classify_block(q0, q1, k0, k1, causal, vl) == \
            sch.classify_block(q0, q1, k0, k1, causal, vl), (q0, q1, k0, k1, causal, vl)
    # negative valid_len means no padding
    assert ra.classify_block(0, 4, 0, 4, False, -1) == ra.RA_FULL


def test_device_entry_points_validate_before_launch(lib):
    """Validation errors come back synchronously without touching a GPU
    (null pointers, bad sizes, unsupported head dimension, bad rank)."""
    import ctypes
    null = None
    # unsupported head dimension
    st = lib.ra_block_attn_fwd(null, null, null, 1, 4, 4, 1, 96, ra.RA_BF16, 0.0, 0, 0,
                               0, -1, null, null, null, null, null)
    assert st == 5 and b"96" in lib.ra_last_error()
    # null pointers with non-empty sizes
    st = lib.ra_block_attn_fwd(null, null, null, 1, 4, 4, 1, 64, ra.RA_BF16, 0.0, 0, 0,
                               0, -1, null, null, null, null, null)
    assert st == 1
    # empty problem: nothing to do, OK without pointers
    st = lib.ra_block_attn_fwd(null, null, null, 0, 4, 4, 1, 64, ra.RA_BF16, 0.0, 0, 0,
                               0, -1, null, null, null, null, null)
    assert st == 0
    # ring: rank >= P and P > RA_MAX_P
    arr = (ctypes.c_void_p * 2)()
    st = lib.ra_ring_attn_fwd(null, arr, arr, 1, 16, 1, 64, 2, 2, ra.RA_BF16, 0.0, 0,
                              -1, null, null, null)
    assert st == 4
    st = lib.ra_ring_attn_fwd(null, arr, arr, 1, 16, 1, 64, 65, 0, ra.RA_BF16, 0.0, 0,
                              -1, null, null, null)
    assert st == 4
    # permutations: S not divisible by P names the padded length; H % P
    st = lib.ra_seq2head(ctypes.c_void_p(16), ctypes.c_void_p(1 << 40), 4, 1, 3002, 8, 64, 2, null)
    assert st == 2 and b"3008" in lib.ra_last_error()
    st = lib.ra_seq2head(ctypes.c_void_p(16), ctypes.c_void_p(1 << 40), 4, 1, 3008, 6, 64, 2, null)
    assert st == 2
    st = lib.ra_head2seq(ctypes.c_void_p(16), ctypes.c_void_p(1 << 40), 4, 1, 3008, 8, 64, 3, null)
    assert st == 3
    # zigzag: rows per rank not two chunks of a multiple of 64; rank >= P;
    # P above RA_MAX_P / 2
    st = lib.ra_zigzag_attn_fwd(null, arr, arr, 1, 96, 1, 64, 2, 0, ra.RA_BF16, 0.0, 1,
                                -1, null, null, null)
    assert st == 2 and b"ra_zigzag_padded_len" in lib.ra_last_error()
    st = lib.ra_zigzag_attn_fwd(null, arr, arr, 1, 128, 1, 64, 2, 2, ra.RA_BF16, 0.0, 1,
                                -1, null, null, null)
    assert st == 4
    st = lib.ra_zigzag_attn_fwd(null, arr, arr, 1, 128, 1, 64, 33, 0, ra.RA_BF16, 0.0, 1,
                                -1, null, null, null)
    assert st == 4
    st = lib.ra_zigzag_attn_fwd(null, arr, arr, 1, 128, 1, 64, 2, 0, ra.RA_BF16, 0.0, 1,
                                -1, null, null, null)
    assert st == 1
    # grouped-query ring: K/V heads must divide H
    st = lib.ra_ring_attn_fwd_gqa(null, arr, arr, 1, 16, 6, 4, 64, 2, 0, ra.RA_BF16, 0.0, 0,
                                  -1, null, null, null)
    assert st == 2 and b"K/V heads" in lib.ra_last_error()
    st = lib.ra_ring_attn_fwd_gqa(null, arr, arr, 1, 16, 6, 0, 64, 2, 0, ra.RA_BF16, 0.0, 0,
                                  -1, null, null, null)
    assert st == 2
    # ring backward: fp32 inputs unsupported, D, rank, NULL buffers
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 0, ra.RA_FP32,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 5 and b"bf16" in lib.ra_last_error()
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 80, 2, 0, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 5
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 3, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 4
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 0, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 1
    # one-round backward: fp32 unsupported, D, NULL, empty
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 64, ra.RA_FP32,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 5 and b"bf16" in lib.ra_last_error()
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 96, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 5 and b"96" in lib.ra_last_error()
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 64, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 1
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 0, 1, 64, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 0
    # merge: unsupported D, unknown dtype
    st = lib.ra_ring_merge(null, null, null, null, 1, 4, 1, 12, null, ra.RA_FP32, null)
    assert st == 5
    st = lib.ra_ring_merge(null, null, null, null, 1, 4, 1, 64, null, 7, null)
    assert st == 3


def test_binding_refuses_cpu_tensors(lib):
    """The binding never falls back to a CPU computation."""
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ra.block_attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        ra.seq2head(torch.zeros(2, 1, 4, 2, 8, dtype=torch.bfloat16))
