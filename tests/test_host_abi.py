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
    assert ra.abi_version() == 2


def test_kernel_option(lib):
    assert ra.get_attn_kernel() == ra.RA_KERNEL_AUTO
    for c in (ra.RA_KERNEL_ROWMAX, ra.RA_KERNEL_AUTO):
        ra.set_attn_kernel(c)
        assert ra.get_attn_kernel() == c
    for bad in (2, 5, 7, -1):
        with pytest.raises(RuntimeError):
            ra.set_attn_kernel(bad)
    assert ra.get_attn_kernel() == ra.RA_KERNEL_AUTO
    assert ra.get_attn_waves() == 0
    for wv in (4, 8, 0):
        ra.set_attn_waves(wv)
        assert ra.get_attn_waves() == wv
    for bad in (1, 2, 16, -4):
        with pytest.raises(RuntimeError):
            ra.set_attn_waves(bad)
    assert ra.get_attn_waves() == 0
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


def _plan_model(B, Sb, H, D, P, rank, causal=False, valid=-1, ns=0):
    """Independent model of the split plan: runs per 128-row query tile so
    that the workgroups fit 512 slots once, each at least 8 of the longest
    query tile's visited 64-key tiles; 1 when the single pass fills them."""
    S = P * Sb
    valid = S if valid < 0 or valid > S else valid
    n_qt = -(-Sb // 128)
    base = B * H * n_qt
    if base == 0:
        return 1, 0
    if ns <= 0:
        if base >= 512:
            return 1, 0
        src, cls = sch.ring_schedule(P, rank, Sb, causal, valid)
        starts = [j * Sb for j, c in zip(src, cls) if c != ra.RA_SKIP]
        max_t = 0
        for qt in range(n_qt):
            q_hi = rank * Sb + min((qt + 1) * 128, Sb) - 1
            lim = min(valid - 1, q_hi) if causal else valid - 1
            t = sum(0 if lim < k0 else min(-(-Sb // 64), (lim - k0) // 64 + 1) for k0 in starts)
            max_t = max(max_t, t)
        ns = min(512 // base, max_t // 8)
    if ns <= 1:
        return 1, 0
    return ns, base * ns * 128 * (D + 1)


def test_split_plan(lib):
    """The split plan against an independent model: the DiT shard (192
    workgroups of 128 rows, 64 tiles each) gets two runs per query tile (384
    workgroups); the long-context share fills the chip and is not split;
    forced counts, causal ranks and padding; -1 on bad sizes."""
    assert ra.ring_split_plan(1, 1024, 24, 128, 4, 0) == (2, 192 * 2 * 128 * 129)
    assert ra.ring_split_plan(1, 16384, 64, 128, 8, 3, causal=True) == (1, 0)
    cases = [(1, 1024, 24, 128, 4, r, c, -1, n) for r in range(4) for c in (False, True)
             for n in (0, 1, 3, 7)]
    cases += [(2, 752, 16, 64, 4, r, True, 3000, n) for r in range(4) for n in (0, 5)]
    cases += [(1, 512, 4, 64, 8, r, c, -1, 0) for r in range(8) for c in (False, True)]
    cases += [(1, 128 * 70, 2, 128, 2, 0, False, -1, 0)]
    for B, Sb, H, D, P, r, c, vl, n in cases:
        assert ra.ring_split_plan(B, Sb, H, D, P, r, c, vl, n) == \
            _plan_model(B, Sb, H, D, P, r, c, vl, n), (B, Sb, H, D, P, r, c, vl, n)
    with pytest.raises(ValueError):
        ra.ring_split_plan(1, 16, 1, 64, 0, 0)
    with pytest.raises(ValueError):
        ra.ring_split_plan(1, 16, 1, 96, 2, 0)


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
    # ring backward: unknown dtype, fp32 validated like bf16, D, rank, NULL buffers
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 0, 7,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 3 and b"dtype" in lib.ra_last_error()
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 0, ra.RA_FP32,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 1
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 80, 2, 0, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 5
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 3, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 4
    st = lib.ra_ring_attn_bwd(null, arr, arr, null, null, null, 1, 16, 1, 64, 2, 0, ra.RA_BF16,
                              0.0, 0, -1, null, arr, arr, null, null)
    assert st == 1
    # split ring: run count below 1
    st = lib.ra_ring_attn_fwd_split(null, arr, arr, 1, 128, 1, 1, 64, 2, 0, ra.RA_BF16, 0.0, 0,
                                    -1, 0, null, 0, null, null, null)
    assert st == ra.RA_ERR_RANGE and b"nsplit" in lib.ra_last_error()
    # one-round backward: fp32 validated like bf16 (NULL), D, NULL, empty
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 64, ra.RA_FP32,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 1
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 96, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 5 and b"96" in lib.ra_last_error()
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 16, 1, 64, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 1
    st = lib.ra_block_attn_bwd(null, null, null, null, null, null, 1, 16, 0, 1, 64, ra.RA_BF16,
                               0.0, 0, 0, 0, -1, null, null, null, null, null)
    assert st == 0
    # zigzag backward: rows per rank not two chunks of a multiple of 64; fp32
    st = lib.ra_zigzag_attn_bwd(null, arr, arr, null, null, null, 1, 96, 1, 64, 2, 0, ra.RA_BF16,
                                0.0, 1, -1, null, arr, arr, null, null)
    assert st == 2 and b"ra_zigzag_padded_len" in lib.ra_last_error()
    st = lib.ra_zigzag_attn_bwd(null, arr, arr, null, null, null, 1, 128, 1, 64, 2, 0, ra.RA_FP32,
                                0.0, 1, -1, null, arr, arr, null, null)
    assert st == 1  # fp32 accepted; the NULL buffers are refused
    st = lib.ra_zigzag_attn_bwd(null, arr, arr, null, null, null, 1, 128, 1, 64, 2, 0, ra.RA_BF16,
                                0.0, 1, -1, null, arr, arr, null, null)
    assert st == 1
    # grouped-query backward: K/V heads must divide H
    st = lib.ra_ring_attn_bwd_gqa(null, arr, arr, null, null, null, 1, 16, 6, 4, 64, 2, 0,
                                  ra.RA_BF16, 0.0, 0, -1, null, arr, arr, null, null)
    assert st == 2 and b"K/V heads" in lib.ra_last_error()
    # packed-sample backward: bad boundary table
    import ctypes as ct
    bad = (ct.c_longlong * 3)(0, 10, 5)
    st = lib.ra_ring_attn_bwd_varlen(null, arr, arr, null, null, null, 16, 1, 64, 2, 0,
                                     ra.RA_BF16, 0.0, 1, bad, 2, null, arr, arr, null, null)
    assert st == 2 and b"increase" in lib.ra_last_error()
    # accumulate mode: unsupported D, missing accumulators, misaligned final
    # output, negative positions; an empty problem is a no-op
    st = lib.ra_block_attn_fwd_acc(null, null, null, 1, 4, 4, 1, 96, ra.RA_BF16, 0.0, 0, 0,
                                   0, -1, null, null, null, null)
    assert st == 5 and b"96" in lib.ra_last_error()
    st = lib.ra_block_attn_fwd_acc(ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   ctypes.c_void_p(256), 1, 4, 4, 1, 64, ra.RA_BF16, 0.0, 0, 0,
                                   0, -1, null, null, null, null)
    assert st == 1 and b"ra_block_attn_fwd_acc" in lib.ra_last_error()
    st = lib.ra_block_attn_fwd_acc(ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   ctypes.c_void_p(256), 1, 4, 4, 1, 64, ra.RA_BF16, 0.0, 0, 0,
                                   0, -1, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   ctypes.c_void_p(258), null)
    assert st == 2 and b"aligned" in lib.ra_last_error()
    st = lib.ra_block_attn_fwd_acc(ctypes.c_void_p(256), ctypes.c_void_p(256),
                                   ctypes.c_void_p(256), 1, 4, 4, 1, 64, ra.RA_BF16, 0.0, -1, 0,
                                   0, -1, ctypes.c_void_p(256), ctypes.c_void_p(256), null, null)
    assert st == 4
    st = lib.ra_block_attn_fwd_acc(null, null, null, 1, 0, 4, 1, 64, ra.RA_BF16, 0.0, 0, 0,
                                   0, -1, null, null, null, null)
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
    acc = torch.zeros(1, 4, 1, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        ra.block_attn_fwd_acc(q, q, q, acc, torch.zeros(1, 4, 1))


def test_binding_checks_output_buffers_before_the_library(lib):
    """Caller-supplied outputs are checked for shape, dtype and device before
    any pointer reaches the library, which cannot see buffer sizes."""
    import torch
    like = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    good = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    for bad, what in ((torch.zeros(1, 3, 2, 64, dtype=torch.bfloat16), "shape"),
                      (torch.zeros(1, 4, 2, 64, dtype=torch.float32), "dtype"),
                      (torch.zeros(1, 4, 2, 32, dtype=torch.bfloat16), "shape")):
        with pytest.raises(ValueError, match=r"\(1, 4, 2, 64\)"):
            ra._out(bad, "out", like.shape, like.dtype, like)
    # a well-formed CPU buffer passes the shape check and is then refused as
    # a host buffer
    with pytest.raises(ValueError, match="GPU"):
        ra._out(good, "out", like.shape, like.dtype, like)


# ------------------------------------------------------------ lockstep order
def _simulate(order, work, n_cu=32):
    """Dispatch one XCD's workgroups in order, each onto the first CU to
    become free, in units of key-tile steps (every step the same time).
    work(bh, qt, rot) -> (first part, second part, index of the full part).
    Returns per workgroup (start of its full-block part, end)."""
    import heapq
    free = [(0, c) for c in range(n_cu)]
    heapq.heapify(free)
    out = {}
    for key in order:
        t, c = heapq.heappop(free)
        a, b, full_first = work(*key)
        full_start = t if full_first else t + a
        end = t + a + b
        out[key] = (full_start, end)
        heapq.heappush(free, (end, c))
    return out


@pytest.mark.parametrize("Q,BH,later_rot,case", [
    (64, 16, 1, "ring"),         # 256-row tiles of a 16384-row share, 16 heads
    (128, 8, 1, "ring"),         # two chunk pairs per head
    (64, 8, 2, "zigzag0"),       # zigzag rank 0 of P = 8 (later half sees 15 whole chunks)
    (64, 8, 2, "zigzag7"),       # zigzag rank 7 (8 whole chunks for the later half, 7 for the earlier)
])
def test_lockstep_order_walks_in_step(lib, Q, BH, later_rot, case):
    """The lockstep order (ra_lockstep_order): a bijection onto (head, tile);
    each XCD takes whole heads; within a head the later 32-tile chunk carries
    the rotation and the earlier chunk follows in decreasing tile order.  In a
    model with one key tile per step and one workgroup per CU, the 32
    workgroups of each chunk pair on an XCD all run their full-block part
    over the same steps, and the earlier chunk's all finish together, when
    the pair's last workgroup does ([RA] §3.4: tile qt of 256 rows sees
    4 (qt + 1) diagonal key tiles of 64)."""
    ok, bh, qt, rot = ra.lockstep_order(Q, BH, later_rot)
    assert ok
    n = Q * BH
    assert sorted(zip(bh, qt)) == [(h, t) for h in range(BH) for t in range(Q)]
    per = n // 8
    for x in range(8):
        ids = list(range(x, n, 8))
        heads = [bh[i] for i in ids]
        assert heads == sorted(heads)  # whole heads, one after another
        assert set(heads) == set(range(x * per // Q, (x + 1) * per // Q))
        for h in set(heads):
            tiles = [(qt[i], rot[i]) for i in ids if bh[i] == h]
            for p in range(Q // 64):
                later, earlier = tiles[64 * p:64 * p + 32], tiles[64 * p + 32:64 * p + 64]
                top = Q - 64 * p
                assert sorted(t for t, _ in later) == list(range(top - 32, top))
                assert all(r == later_rot for _, r in later)
                assert [t for t, _ in earlier] == list(range(top - 33, top - 65, -1))
                assert all(r == 0 for _, r in earlier)

        def work(h, t, r, Q=Q):
            if case == "ring":      # full blocks F, diagonal 4(t+1)
                full, diag = 768, 4 * (t + 1)
            else:                   # zigzag: the two halves of the share
                later = t >= Q // 2
                i = t - Q // 2 if later else t
                wholes = {"zigzag0": (15, 0), "zigzag7": (8, 7)}[case][0 if later else 1]
                full, diag = 128 * wholes, 4 * (i + 1)
            return (full, diag, True) if r else (diag, full, False)

        sim = _simulate([(bh[i], qt[i], rot[i]) for i in ids], work)
        for h in set(heads):
            keys = [(bh[i], qt[i], rot[i]) for i in ids if bh[i] == h]
            for p in range(Q // 64):
                pair = keys[64 * p:64 * p + 64]
                later, earlier = pair[:32], pair[32:]
                assert len({sim[k][0] for k in later}) == 1
                if case != "zigzag0":  # the earlier half of rank 0 has no full part
                    assert len({sim[k][0] for k in earlier}) == 1
                # the earlier chunk's workgroups all end when the pair's
                # last one does, so the next pair starts in step
                ends = {sim[k][1] for k in earlier}
                assert len(ends) == 1 and ends == {max(sim[k][1] for k in pair)}


def test_lockstep_order_declines_other_shapes(lib):
    assert not ra.lockstep_order(32, 16)[0]    # half a chunk pair per head
    assert not ra.lockstep_order(64, 12)[0]    # heads do not split evenly over 8 XCDs
    with pytest.raises(ValueError):
        ra.lockstep_order(0, 8)
