"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (written here, from the pages): bf16 inputs with fp32
accumulation -- max_abs_err <= 1e-2 and cosine > 0.999 against the
full-sequence reference (juejin post §二 table, §三 check [2]); fp32 --
max_abs_err <= 1e-5 (fused-operator precision page §3.4, fp32 tier);
layout permutations -- bit-exact (same page: integer / bitwise data exact).
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.attention import _f64

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_ulysses_sequence_amd")

BF16_ATOL, BF16_COS, FP32_ATOL = 1e-2, 0.999, 1e-5
# lse of a bf16 call: P is rounded to bf16 (relative error <= 2^-8) before it
# enters P V, and the denominator sums those same rounded weights so that O
# stays an exact convex combination of V rows; the log-sum-exp therefore
# carries up to ln(1 + 2^-8) = 3.9e-3 of that rounding (plus fp32 noise).
LSE_BF16_ATOL = 4e-3


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (torch.cuda.is_available() is False)")
    if not os.path.exists(ra.LIB_PATH):
        pytest.fail("libringattn.so is not built")
    ra.lib()
    yield
    torch.cuda.synchronize()


@pytest.fixture(params=["auto", "rowmax-w4", "auto-w8", "rowmax-w8"])
def variant(request):
    """Run a bf16 test under each kernel configuration (all compute the same
    function): the way of keeping the row max (the reference set once per
    row with tiles over the weight bound redone, or the row max of every
    tile) and the waves per workgroup (the library's choice, 4 or 8)."""
    mx, _, wv = request.param.partition("-")
    ra.set_attn_kernel({"auto": ra.RA_KERNEL_AUTO, "rowmax": ra.RA_KERNEL_ROWMAX}[mx])
    ra.set_attn_waves({"": 0, "w4": 4, "w8": 8}[wv])
    yield request.param
    ra.set_attn_kernel(ra.RA_KERNEL_AUTO)
    ra.set_attn_waves(0)


def check_bf16(got, ref, what):
    c = oracle.compare(got, ref)
    say(what, {k: f"{v:.3e}" for k, v in c.items()})
    assert np.all(np.isfinite(_f64(got)))
    assert c["max_abs_err"] <= BF16_ATOL, (what, c)
    assert c["cos"] > BF16_COS, (what, c)
    return c


def check_fp32(got, ref, what, atol=FP32_ATOL):
    c = oracle.compare(got, ref)
    say(what, {k: f"{v:.3e}" for k, v in c.items()})
    assert c["max_abs_err"] <= atol, (what, c)
    return c


def check_lse(got, ref, what="lse", atol=LSE_BF16_ATOL):
    """lse within its tolerance; the measured error is printed so that runs
    record how much of the derived bound is used."""
    e = oracle.max_abs_err(got, ref)
    say(what, f"lse max_abs_err {e:.3e} (bound {atol:.0e})")
    assert e <= atol, (what, e)
    return e


def blocks_of(x, P):
    """P contiguous sequence blocks of a [B, S, H, D] tensor (the ring buffers)."""
    Sb = x.shape[1] // P
    return [x[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(P)]


def oracle_share(q, k, v, w, rank, rows=None, heads=None):
    """Oracle attention of rank's share over the global K/V (per head to keep
    host memory small).  Returns o [B, R, H', D], lse [B, R, H']."""
    Sb = w.block_len
    heads = range(w.H) if heads is None else heads
    q_r = q[:, rank * Sb:(rank + 1) * Sb]
    klim = (rank + 1) * Sb if w.causal else k.shape[1]
    os_, ls_ = [], []
    for h in heads:
        o, lse, _, _ = oracle.attention(q_r[:, :, h:h + 1], k[:, :klim, h:h + 1],
                                        v[:, :klim, h:h + 1], causal=w.causal,
                                        q_pos0=rank * Sb, k_pos0=0, valid_len=w.S,
                                        rows=rows)
        os_.append(o)
        ls_.append(lse)
    return np.concatenate(os_, axis=2), np.concatenate(ls_, axis=2)


def real_rows(w, rank):
    """Rows of rank's share that are real tokens (pad queries are discarded)."""
    Sb = w.block_len
    n = max(0, min(Sb, w.S - rank * Sb))
    return np.arange(n)


# ------------------------------------------------------------ worked example
def test_worked_example_through_abi():
    """Tutorial §04 example: D zero-padded 2 -> 64 (scores unchanged), scale
    1/sqrt(2) passed explicitly, two ranks with K/V blocks of two rows."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "ring_tutorial_worked_example.json")))
    def pad(x):
        t = torch.zeros(1, 4, 1, 64, dtype=torch.float32)
        t[0, :, 0, :2] = torch.tensor(x, dtype=torch.float32)
        return t.cuda()
    q, k, v = pad(g["q"]), pad(g["k"]), pad(g["v"])
    kb, vb = blocks_of(k, 2), blocks_of(v, 2)
    outs = []
    for r in range(2):
        say("worked example rank", r)
        o, _ = ra.ring_attn_fwd(q[:, 2 * r:2 * r + 2].contiguous(), kb, vb, r,
                                scale=1 / math.sqrt(2))
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.cat(outs, 1).cpu()
    np.testing.assert_allclose(o[0, 0, 0, :2].numpy(), g["full_row0"], atol=2e-6)
    assert torch.all(o[..., 2:] == 0)
    full, _, _, _ = oracle.attention(q[..., :2].cpu(), k[..., :2].cpu(), v[..., :2].cpu())
    check_fp32(o[..., :2], full, "worked example all rows")


# ------------------------------------------------------------ C1 tiny fp32
@pytest.mark.parametrize("path", ["fused", "composable"])
def test_tiny_fp32_ring(path):
    w = W.TINY_FP32
    q, k, v = W.make_qkv(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    for r in w.ranks:
        say(w.name, path, "rank", r)
        q_r = qg[:, r * w.block_len:(r + 1) * w.block_len].contiguous()
        fn = ra.ring_attn_fwd if path == "fused" else ra.ring_attn_composable
        o, lse = fn(q_r, kb, vb, r)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle_share(q, k, v, w, r)
        check_fp32(o.cpu(), ref_o, f"{w.name} {path} r{r} O")
        check_fp32(lse.cpu(), ref_lse, f"{w.name} {path} r{r} lse", atol=1e-5)
        loc = oracle.local_only_attention(q_r.cpu(), kb[r].cpu(), vb[r].cpu(),
                                          pos0=r * w.block_len)
        assert oracle.max_abs_err(o.cpu(), loc) > 0


# ------------------------------------------------------------ C2 DiT shard
@pytest.fixture(scope="module")
def dit():
    w = W.DIT_SHARD
    q, k, v = W.make_qkv(w)
    return w, (q, k, v), (q.cuda(), k.cuda(), v.cuda())


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_dit_shard_fused(dit, rank, variant):
    w, (q, k, v), (qg, kg, vg) = dit
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    q_r = qg[:, rank * w.block_len:(rank + 1) * w.block_len].contiguous()
    say(w.name, "fused rank", rank)
    o, lse = ra.ring_attn_fwd(q_r, kb, vb, rank)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle_share(q, k, v, w, rank)
    check_bf16(o.cpu(), ref_o, f"{w.name} r{rank} O")
    check_lse(lse.cpu(), ref_lse)
    # communication really happened: differs from local-only attention
    loc = oracle.local_only_attention(q_r.cpu(), kb[rank].cpu(), vb[rank].cpu())
    assert oracle.max_abs_err(o.cpu(), loc) > 0
    assert oracle.cosine(o.cpu(), loc) < BF16_COS


def test_dit_shard_composable_matches(dit, variant):
    w, (q, k, v), (qg, kg, vg) = dit
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    r = 2
    q_r = qg[:, r * w.block_len:(r + 1) * w.block_len].contiguous()
    say(w.name, "composable rank", r)
    o_c, lse_c = ra.ring_attn_composable(q_r, kb, vb, r)
    o_f, lse_f = ra.ring_attn_fwd(q_r, kb, vb, r)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle_share(q, k, v, w, r)
    check_bf16(o_c.cpu(), ref_o, f"{w.name} composable r{r}")
    check_lse(lse_c.cpu(), ref_lse)
    assert oracle.max_abs_err(o_c.cpu(), o_f.cpu()) <= BF16_ATOL


def test_dit_shard_deterministic(dit, variant):
    """No atomics on the path: two runs are bitwise identical."""
    w, _, (qg, kg, vg) = dit
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    q_r = qg[:, :w.block_len].contiguous()
    say(w.name, "determinism")
    a, la = ra.ring_attn_fwd(q_r, kb, vb, 0)
    b, lb = ra.ring_attn_fwd(q_r, kb, vb, 0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la, lb)


def test_block_attn_partials_and_stats(dit, variant):
    """One round (block_attn_fwd): o, lse, m, l against the oracle, with
    global positions; then merging all rounds gives the ring result."""
    w, (q, k, v), (qg, kg, vg) = dit
    r, Sb = 1, w.block_len
    q_r = qg[:, r * Sb:(r + 1) * Sb].contiguous()
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    j = 3
    say(w.name, "block_attn_fwd block", j)
    o, lse, m, l = ra.block_attn_fwd(q_r, kb[j], vb[j], q_pos0=r * Sb, k_pos0=j * Sb)
    torch.cuda.synchronize()
    ro, rl, rm, rll = oracle.attention(q[:, r * Sb:(r + 1) * Sb], k[:, j * Sb:(j + 1) * Sb],
                                       v[:, j * Sb:(j + 1) * Sb])
    check_bf16(o.cpu(), ro, "block_attn o")
    check_lse(lse.cpu(), rl)
    assert oracle.max_abs_err(m.cpu(), rm) <= 1e-4 * max(1.0, float(np.abs(rm).max()))
    # l sums bf16-rounded weights: relative error up to 2^-8
    np.testing.assert_allclose(l.cpu().numpy(), rll, rtol=4e-3)
    np.testing.assert_allclose(lse.cpu().numpy(),
                               m.cpu().numpy() + np.log(l.cpu().numpy()), atol=1e-5)


# ------------------------------------------------------------ accumulate mode
@pytest.mark.parametrize("dtype,D,causal", [(torch.bfloat16, 128, True), (torch.bfloat16, 64, False),
                                            (torch.bfloat16, 128, False), (torch.float32, 64, True)])
def test_block_attn_fwd_acc_rounds(dtype, D, causal):
    """ra_block_attn_fwd_acc one round at a time, in a scrambled order, from
    an empty start (o = 0, lse = -inf): a query shard of 200 rows (global
    rows 300..499) against four K/V blocks of uneven, ragged lengths (130,
    170, 220, 180 keys; real length 610, the rest padding).  After every
    fold the running (o_acc, lse_acc) against the oracle's lse_combine of
    the plain per-block attentions; the last fold writes the output in the
    input dtype and must leave o_acc as it was.  Causal: the block after
    every query is SKIP and leaves the partial bitwise unchanged."""
    B, H, Sq, q0, valid = 2, 3, 200, 300, 610
    bounds = [0, 130, 300, 520, 700]
    S = bounds[-1]
    q, k, v = (W.random_tensor((B, S, H, D), seed=s_, dtype=dtype) for s_ in (61, 62, 63))
    q = q[:, q0:q0 + Sq].contiguous()
    qg = q.cuda()
    o_acc = torch.zeros((B, Sq, H, D), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((B, Sq, H), -math.inf, dtype=torch.float32, device="cuda")
    ref_o = ref_l = None
    order = [2, 0, 3, 1]
    atol, latol = (BF16_ATOL, LSE_BF16_ATOL) if dtype == torch.bfloat16 else (FP32_ATOL, 1e-5)
    for n, j in enumerate(order):
        a_, b_ = bounds[j], bounds[j + 1]
        kb, vb = k[:, a_:b_].contiguous(), v[:, a_:b_].contiguous()
        last = n == len(order) - 1
        final = torch.full((B, Sq, H, D), 7.0, dtype=dtype, device="cuda") if last else None
        before = o_acc.clone(), lse_acc.clone()
        say("block_attn_fwd_acc", dtype, D, causal, "keys", a_, b_, "final" if last else "")
        ra.block_attn_fwd_acc(qg, kb.cuda(), vb.cuda(), o_acc, lse_acc, q_pos0=q0, k_pos0=a_,
                              causal=causal, valid_len=valid, out_final=final)
        torch.cuda.synchronize()
        bo, bl, _, _ = oracle.attention(q, kb, vb, causal=causal, q_pos0=q0, k_pos0=a_,
                                        valid_len=valid)
        ref_o, ref_l = (bo, bl) if ref_o is None else oracle.lse_combine(ref_o, ref_l, bo, bl)
        got_o = final if last else o_acc
        if causal and a_ > q0 + Sq - 1:
            assert torch.equal(o_acc, before[0]) and torch.equal(lse_acc, before[1])
        if last:
            assert torch.equal(o_acc, before[0]), "o_acc written in the final round"
        c = oracle.compare(got_o.float().cpu(), ref_o)
        say("  o", {kk: f"{vv:.3e}" for kk, vv in c.items()})
        assert c["max_abs_err"] <= atol, c
        gl = lse_acc.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.max(np.abs(gl[fin] - ref_l[fin]), initial=0.0) <= latol
    full, full_l, _, _ = oracle.attention(q, k, v, causal=causal, q_pos0=q0, valid_len=valid)
    check = check_bf16 if dtype == torch.bfloat16 else check_fp32
    check(final.float().cpu(), full, f"acc rounds {dtype} D={D} causal={causal} final")


# ------------------------------------------------------------ split ring
@pytest.mark.parametrize("causal,D,pad,Hkv,P", [(False, 128, 0, 4, 4), (True, 128, 0, 4, 4),
                                                (True, 64, 37, 4, 4), (True, 128, 0, 2, 4),
                                                (False, 64, 0, 4, 8)])
def test_split_ring_all_ranks(causal, D, pad, Hkv, P):
    """The split ring (each 128-row query tile's visited-tile sequence cut
    into near-equal runs computed by separate workgroups, fp32 partials
    merged by log-sum-exp) for 2 to more runs than some tiles have (empty
    runs) and the plan's own count, on every rank, against the oracle and
    against the single pass (within the bf16 budget: each run rounds its
    weights against its own reference max)."""
    B, S, H = 1, 2048, 4
    Sb, valid = S // P, S - pad
    q, k, v = (W.random_tensor((B, S, h_, D), seed=s_) for s_, h_ in ((61, H), (62, Hkv), (63, Hkv)))
    if pad:
        for x in (q, k, v):
            x[:, valid:] = 0
    kb, vb = blocks_of(k.cuda(), P), blocks_of(v.cuda(), P)
    kk = k.repeat_interleave(H // Hkv, dim=2)
    vv = v.repeat_interleave(H // Hkv, dim=2)
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous().cuda()
        ref_o, ref_lse, _, _ = oracle.attention(q[:, r * Sb:(r + 1) * Sb], kk, vv, causal=causal,
                                                q_pos0=r * Sb, valid_len=valid)
        rows = np.arange(max(0, min(Sb, valid - r * Sb)))
        o1, l1 = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid, split=1)
        auto, _ = ra.ring_split_plan(B, Sb, H, D, P, r, causal, valid)
        for ns in sorted({2, 3, 5, 40, auto} - {1}):
            say("split ring", causal, D, pad, Hkv, P, "rank", r, "runs", ns)
            o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid, split=ns)
            torch.cuda.synchronize()
            check_bf16(o.cpu()[:, rows], ref_o[:, rows], f"runs {ns} r{r} O")
            check_lse(lse.cpu()[:, rows], ref_lse[:, rows])
            # against the single pass: a bf16 step of the output (2^-7
            # relative at most) plus the weights' rounding
            d = (o.float() - o1.float()).abs()
            assert bool((d <= 2.0 ** -7 * o1.float().abs() + 2e-3).all()), float(d.max())
            assert float((lse - l1).abs().max()) <= LSE_BF16_ATOL


def test_noalloc_split_under_graph_capture():
    """ra_ring_attn_fwd_split_noalloc is for callers that cannot allocate,
    such as code under HIP graph capture: captured once (it allocates nothing
    and records no memset), replayed three times with the library's own eager
    work and synchronisations in between (an eager call on another share that
    overwrites the same scratch, and fills of the outputs), every replay bit-
    identical to the eager result of the captured call."""
    B, S, H, D, P, rank = 1, 4096, 24, 128, 4, 0
    q, k, v = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (81, 82, 83))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    Sb = S // P
    q_r = q[:, rank * Sb:(rank + 1) * Sb].contiguous()
    runs, _ = ra.ring_split_plan(B, Sb, H, D, P, rank, False, -1, 0)
    assert runs > 1, "the case must exercise the split"
    o_e = torch.empty_like(q_r)
    l_e = torch.empty((B, Sb, H), dtype=torch.float32, device="cuda")
    ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o_e, l_e)
    # another share for the eager calls between replays (same scratch)
    q2, k2, v2 = (W.random_tensor((1, 1024, 4, 64), seed=s_, device="cuda") for s_ in (84, 85, 86))
    kb2, vb2 = blocks_of(k2, 2), blocks_of(v2, 2)
    q2_r = q2[:, 512:].contiguous()
    o2 = torch.empty_like(q2_r)
    o_g = torch.empty_like(q_r)
    l_g = torch.empty_like(l_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o_g, l_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("noalloc split: capture")
    with torch.cuda.graph(graph):
        ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o_g, l_g)
    for rep in range(3):
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        ra.ring_attn_fwd_split_noalloc(q2_r, kb2, vb2, 1, o2, causal=True, nsplit=2)
        torch.cuda.synchronize()
        say("noalloc split: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), rep
        assert torch.equal(l_g.view(torch.int32), l_e.view(torch.int32)), rep


def test_explicit_stream_orders_default_buffers():
    """Calls given stream= allocate and zero-fill their default outputs and
    scratch on that stream: with the current stream still busy (and the
    side stream not waiting for it), the backward (zero-filled dq / dk / dv,
    statistics scratch) and a split forward (partial workspace) on the side
    stream give the same bits as on the current stream."""
    B, S, H, D, P, rank = 1, 2048, 4, 64, 2, 1
    q, k, v, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (91, 92, 93, 94))
    Sb = S // P
    q_r, do_r = q[:, rank * Sb:].contiguous(), do[:, rank * Sb:].contiguous()
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    o_r, lse_r = ra.ring_attn_fwd(q_r, kb, vb, rank, causal=True)
    ref_b = ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, rank, causal=True)
    ref_f = ra.ring_attn_fwd(q_r, kb, vb, rank, split=2)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    # keep the current stream busy for a while (fp32 products, no transposed views)
    a = torch.randn(4096, 4096, device="cuda")
    for _ in range(12):
        a = torch.mm(a, a) * 1e-3
    say("explicit stream: calls on the side stream while the current one is busy")
    got_b = ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, rank, causal=True, stream=side)
    got_f = ra.ring_attn_fwd(q_r, kb, vb, rank, split=2, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(got_b[0], ref_b[0])
    for j in range(P):
        assert torch.equal(got_b[1][j], ref_b[1][j]), j
        assert torch.equal(got_b[2][j], ref_b[2][j]), j
    assert torch.equal(got_f[0].view(torch.int16), ref_f[0].view(torch.int16))
    assert torch.equal(got_f[1].view(torch.int32), ref_f[1].view(torch.int32))
    assert torch.isfinite(a).all()


def test_split_ring_errors():
    """A run count below one is refused; a split without workspace or with
    too small a workspace is refused before any launch."""
    import ctypes
    q = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16, device="cuda")
    kb = [q, q]
    with pytest.raises(ValueError):
        ra.ring_attn_fwd(q, kb, kb, 0, split=0)
    arr = (ctypes.c_void_p * 2)(q.data_ptr(), q.data_ptr())
    o = torch.empty_like(q)
    lib = ra.lib()
    st = lib.ra_ring_attn_fwd_split(q.data_ptr(), arr, arr, 1, 128, 1, 1, 64, 2, 0, ra.RA_BF16,
                                    0.0, 0, -1, 2, None, 0, o.data_ptr(), None, None)
    assert st == ra.RA_ERR_NULL and b"workspace" in lib.ra_last_error()
    need = ra.ring_split_plan(1, 128, 1, 64, 2, 0, nsplit=2)[1]
    ws = torch.empty(need, dtype=torch.float32, device="cuda")
    st = lib.ra_ring_attn_fwd_split(q.data_ptr(), arr, arr, 1, 128, 1, 1, 64, 2, 0, ra.RA_BF16,
                                    0.0, 0, -1, 2, ws.data_ptr(), need - 1, o.data_ptr(), None,
                                    None)
    assert st == ra.RA_ERR_SHAPE and str(need).encode() in lib.ra_last_error()


# ------------------------------------------------------------ C3 Ulysses
def test_ulysses_layout_and_attention(variant):
    w = W.ULYSSES
    P, Sl, Hl = w.P, w.S // w.P, w.H // w.P
    say(w.name, "generate")
    q, k, v = W.make_qkv(w, device="cuda")
    # the P per-rank sequence shards, stacked rank-major: [P, B, S/P, H, D]
    stack = lambda x: x.view(w.B, P, Sl, w.H, w.D).transpose(0, 1).contiguous()
    qs, ks, vs = stack(q), stack(k), stack(v)
    say(w.name, "seq2head")
    qh, kh, vh = ra.seq2head(qs), ra.seq2head(ks), ra.seq2head(vs)
    torch.cuda.synchronize()
    for src, dst in ((qs, qh), (ks, kh), (vs, vh)):
        assert np.array_equal(dst.cpu().view(torch.int16).numpy(), oracle.seq2head(src.cpu()))
    # local attention on the H/P heads of every rank: the stacked head
    # shards [P, B, S, H/P, D] are one batch of P*B sequences, one ring
    # block (P=1 in the attention call)
    say(w.name, "attention on head shards")
    flat = lambda x: x.view(P * w.B, w.S, Hl, w.D)
    oh, _ = ra.ring_attn_fwd(flat(qh), [flat(kh)], [flat(vh)], 0)
    oh = oh.view(P, w.B, w.S, Hl, w.D)
    say(w.name, "head2seq")
    os_ = ra.head2seq(oh)
    torch.cuda.synchronize()
    assert np.array_equal(os_.cpu().view(torch.int16).numpy(), oracle.head2seq(oh.cpu()))
    assert torch.equal(ra.head2seq(qh).view(torch.int16), qs.view(torch.int16))
    # sampled rows of the final sequence-sharded output vs the oracle
    rows = np.unique(np.concatenate([np.arange(0, w.S, 61), [w.S - 1]]))
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    # every head (each rank's head group and every position inside it)
    ref, _, _, _ = oracle.attention(qc, kc, vc, rows=rows)
    got = os_.transpose(0, 1).reshape(w.B, w.S, w.H, w.D)[:, rows].cpu()
    check_bf16(got, ref, f"{w.name} O sampled rows")


# ------------------------------------------------------------ lockstep order
@pytest.mark.parametrize("D,causal,pad,Hkv", [(128, True, 0, 8), (64, False, 0, 8),
                                              (128, True, 100, 2)])
def test_lockstep_order(D, causal, pad, Hkv):
    """Shares with 64 query tiles of 256 rows per head and heads in eights
    take the lockstep workgroup order in the 8-wave forward and dQ kernels:
    half of each head's query tiles visit the full block first and the
    diagonal block last.  Rank 1 of a P = 2 ring over L = 32768 (H = 8; also
    with 100 padding tokens at the end of the rank's own block and 2 K/V
    heads): every row against the 4-wave kernels (plain ring order), sampled
    rows at a stride co-prime to the tiles (and both sides of the chunk
    boundary at row 8192) against the oracle."""
    B, H, P, Sb = 1, 8, 2, 16384
    S = P * Sb
    valid = S - pad
    q, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (81, 84))
    k, v = (W.random_tensor((B, S, Hkv, D), seed=s_, device="cuda") for s_ in (82, 83))
    for x in (q, k, v):
        x[:, valid:] = 0
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    r = 1
    q_r, do_r = q[:, Sb:].contiguous(), do[:, Sb:].contiguous()
    got = {}
    try:
        for wv in (4, 8):
            ra.set_attn_waves(wv)
            say("lockstep", D, causal, pad, Hkv, "waves", wv)
            o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid)
            g = ra.ring_attn_bwd(q_r, kb, vb, o, do_r, lse, r, causal=causal, valid_len=valid)
            torch.cuda.synchronize()
            got[wv] = (o, lse, g)
    finally:
        ra.set_attn_waves(0)
    o8, l8, g8 = got[8]
    o4, l4, g4 = got[4]
    n = Sb - pad  # the real rows of the share
    check_bf16(o8[:, :n].cpu(), o4[:, :n].cpu().double().numpy(), "lockstep o vs 4 waves")
    assert (l8[:, :n] - l4[:, :n]).abs().max().item() <= LSE_BF16_ATOL
    # the backward of the 8-wave forward's outputs through both dQ forms
    try:
        ra.set_attn_waves(4)
        g48 = ra.ring_attn_bwd(q_r, kb, vb, o8, do_r, l8, r, causal=causal, valid_len=valid)
        torch.cuda.synchronize()
    finally:
        ra.set_attn_waves(0)
    check_grad(g8[0].cpu(), g48[0].cpu().double().numpy(), "lockstep dq vs 4 waves")
    for j in range(P):
        assert torch.equal(g8[1][j], g48[1][j]) and torch.equal(g8[2][j], g48[2][j])
    rows = np.unique(np.concatenate([np.arange(0, n, 127), np.arange(8192 - 3, 8192 + 3),
                                     np.arange(n - 3, n)]))
    kf = oracle.gqa_expand(k.cpu(), H) if Hkv != H else k.cpu()
    vf = oracle.gqa_expand(v.cpu(), H) if Hkv != H else v.cpu()
    ref_o, ref_lse, _, _ = oracle.attention(q_r.cpu(), kf, vf, causal=causal, q_pos0=Sb,
                                            valid_len=valid, rows=rows)
    check_bf16(o8[:, rows].cpu(), ref_o, "lockstep o vs oracle")
    check_lse(l8[:, rows].cpu(), ref_lse)


def test_lockstep_order_zigzag():
    """Causal zigzag shares of two 8192-row chunks (P = 2, L = 32768, H = 8,
    D = 64) take the lockstep order with the later query tiles starting from
    the third block-table entry: every row of both ranks (forward, and dq
    through both dQ forms) against the 4-wave kernels, sampled rows of both
    chunks at a stride co-prime to the tiles against the oracle."""
    B, H, P, c, D = 1, 8, 2, 8192, 64
    S = 2 * P * c
    q, k, v, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (85, 86, 87, 88))
    qs, ks, vs, dos = (zigzag_shares(x, P) for x in (q, k, v, do))
    for r in range(P):
        got = {}
        try:
            for wv in (4, 8):
                ra.set_attn_waves(wv)
                say("lockstep zigzag rank", r, "waves", wv)
                o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=True)
                torch.cuda.synchronize()
                got[wv] = (o, lse)
            o8, l8 = got[8]
            g = {}
            for wv in (4, 8):
                ra.set_attn_waves(wv)
                g[wv] = ra.zigzag_attn_bwd(qs[r], ks, vs, o8, dos[r], l8, r, causal=True)
                torch.cuda.synchronize()
        finally:
            ra.set_attn_waves(0)
        check_bf16(o8.cpu(), got[4][0].cpu().double().numpy(), f"lockstep zigzag r{r} o vs 4 waves")
        assert (l8 - got[4][1]).abs().max().item() <= LSE_BF16_ATOL
        check_grad(g[8][0].cpu(), g[4][0].cpu().double().numpy(), f"lockstep zigzag r{r} dq")
        for j in range(P):
            assert torch.equal(g[8][1][j], g[4][1][j]) and torch.equal(g[8][2][j], g[4][2][j])
        rows = np.unique(np.concatenate([np.arange(0, c, 127), np.arange(c - 3, c)]))
        for half, chunk in enumerate(oracle.zigzag_chunks(P, r)):
            klim = (chunk + 1) * c
            ref_o, ref_l, _, _ = oracle.attention(q[:, chunk * c:(chunk + 1) * c].cpu(),
                                                  k[:, :klim].cpu(), v[:, :klim].cpu(),
                                                  causal=True, q_pos0=chunk * c, rows=rows)
            check_bf16(o8[:, half * c + rows].cpu(), ref_o, f"lockstep zigzag r{r} chunk {chunk}")
            check_lse(l8[:, half * c + rows].cpu(), ref_l)


# ------------------------------------------------------------ C4 long causal
def test_long_context_causal_rank3(variant):
    w = W.LONG_CAUSAL
    r, Sb = 3, w.block_len
    say(w.name, "generate on device")
    q, k, v = W.make_qkv(w, device="cuda")
    kb = [k[:, j * Sb:(j + 1) * Sb] for j in range(w.P)]   # B=1: contiguous views
    vb = [v[:, j * Sb:(j + 1) * Sb] for j in range(w.P)]
    q_r = q[:, r * Sb:(r + 1) * Sb]
    say(w.name, "fused ring rank 3")
    o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    # sampled rows: a stride co-prime to the 128- and 256-row query tiles
    # (so the samples meet every wave and lane position of interior tiles),
    # both edges, and rows around the diagonal tile boundaries (key tile 64)
    rows = np.unique(np.concatenate([
        np.arange(0, Sb, 127), np.arange(0, 32), np.arange(Sb - 32, Sb),
        np.arange(8192 - 3, 8192 + 3), np.arange(127, 130), np.arange(63, 66),
        np.arange(255, 258)]))
    heads = list(range(1, w.H, 3))
    say(w.name, "oracle on", len(rows), "rows x", len(heads), "heads")
    kc = k[:, :(r + 1) * Sb].cpu()
    vc = v[:, :(r + 1) * Sb].cpu()
    ref_o, ref_lse = [], []
    for h in heads:
        o_h, l_h, _, _ = oracle.attention(q_r[:, :, h:h + 1].cpu(), kc[:, :, h:h + 1],
                                          vc[:, :, h:h + 1], causal=True,
                                          q_pos0=r * Sb, k_pos0=0, rows=rows)
        ref_o.append(o_h)
        ref_lse.append(l_h)
    ref_o = np.concatenate(ref_o, 2)
    ref_lse = np.concatenate(ref_lse, 2)
    got = o[:, rows][:, :, heads].cpu()
    check_bf16(got, ref_o, f"{w.name} sampled")
    assert oracle.rel_l2(got, ref_o) < 2e-2
    check_lse(lse[:, rows][:, :, heads].cpu(), ref_lse)


# ------------------------------------------------------------ C5 padded causal
@pytest.fixture(scope="module")
def padded():
    w = W.PADDED_CAUSAL
    q, k, v = W.make_qkv(w)
    return w, (q, k, v), (q.cuda(), k.cuda(), v.cuda())


@pytest.mark.parametrize("path", ["fused", "composable"])
def test_padded_causal_all_ranks(padded, path, variant):
    w, (q, k, v), (qg, kg, vg) = padded
    assert w.S_padded == 3008 and w.block_len == 752
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    fn = ra.ring_attn_fwd if path == "fused" else ra.ring_attn_composable
    for r in w.ranks:
        q_r = qg[:, r * w.block_len:(r + 1) * w.block_len].contiguous()
        say(w.name, path, "rank", r)
        o, lse = fn(q_r, kb, vb, r, causal=True, valid_len=w.S)
        torch.cuda.synchronize()
        rows = real_rows(w, r)
        ref_o, ref_lse = oracle_share(q, k, v, w, r, rows=rows)
        check_bf16(o[:, rows].cpu(), ref_o, f"{w.name} {path} r{r}")
        check_lse(lse[:, rows].cpu(), ref_lse)


def test_padded_skipped_blocks_never_read(padded, variant):
    """Poison the K/V of every block a causal rank skips with NaN: the output
    stays bit-identical.  Poison a visited block: rows that see it change."""
    w, _, (qg, kg, vg) = padded
    kb, vb = blocks_of(kg, w.P), blocks_of(vg, w.P)
    r = 1
    q_r = qg[:, r * w.block_len:(r + 1) * w.block_len].contiguous()
    say(w.name, "poison test")
    base, _ = ra.ring_attn_fwd(q_r, kb, vb, r, causal=True, valid_len=w.S)
    kp = [x.clone() for x in kb]
    vp = [x.clone() for x in vb]
    for j in (2, 3):
        kp[j].fill_(float("nan"))
        vp[j].fill_(float("nan"))
    same, _ = ra.ring_attn_fwd(q_r, kp, vp, r, causal=True, valid_len=w.S)
    vp[0].fill_(1e4)
    diff, _ = ra.ring_attn_fwd(q_r, kp, vp, r, causal=True, valid_len=w.S)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), same.view(torch.int16))
    assert (diff.float() - base.float()).abs().max().item() > 1.0


# ------------------------------------------------------------ zigzag shares
def zigzag_shares(x, P):
    """The P zigzag shares of a [B, S, H, D] tensor (rows at the positions the
    oracle assigns to each rank), each contiguous [B, 2c, H, D]."""
    c = x.shape[1] // (2 * P)
    return [x[:, torch.as_tensor(oracle.zigzag_positions(P, r, c), device=x.device)].contiguous()
            for r in range(P)]


@pytest.mark.parametrize("causal", [True, False])
def test_zigzag_all_ranks(variant, causal):
    """Zigzag shares (chunks r and 2P-1-r), B = 2: every rank's output and
    lse against the oracle's recurrence over the same shares."""
    B, S, H, D, P = 2, 2048, 4, 128, 4
    q, k, v = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (11, 12, 13))
    qs, ks, vs = zigzag_shares(q, P), zigzag_shares(k, P), zigzag_shares(v, P)
    kc, vc = [x.cpu() for x in ks], [x.cpu() for x in vs]
    for r in range(P):
        o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=causal)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle.zigzag_ring_rank(qs[r].cpu(), kc, vc, r, causal=causal)
        check_bf16(o.cpu(), ref_o, f"zigzag causal={causal} r{r}")
        check_lse(lse.cpu(), ref_lse)


def test_zigzag_padded_all_ranks(variant):
    """S = 3000 padded to 3072 (chunks of 384), one K row per (b, h) x8:
    real rows of every rank against the plain definition at their global
    positions (pad queries discarded)."""
    w = W.PADDED_ZIGZAG
    assert w.S_padded == 3072
    q, k, v = W.make_qkv(w)
    qs, ks, vs = (zigzag_shares(x.cuda(), w.P) for x in (q, k, v))
    c = w.S_padded // (2 * w.P)
    full, full_lse, _, _ = oracle.attention(q, k, v, causal=True, valid_len=w.S)
    for r in w.ranks:
        say(w.name, "rank", r)
        o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=True, valid_len=w.S)
        torch.cuda.synchronize()
        pos = oracle.zigzag_positions(w.P, r, c)
        real = np.flatnonzero(pos < w.S)
        check_bf16(o.cpu()[:, real], full[:, pos[real]], f"{w.name} r{r}")
        check_lse(lse.cpu()[:, real], full_lse[:, pos[real]])


def test_zigzag_fp32():
    """fp32 inputs through the fp32 kernel: every rank to 1e-5."""
    B, S, H, D, P = 1, 1024, 2, 64, 2
    q, k, v = (W.random_tensor((B, S, H, D), dtype=torch.float32, seed=s_, device="cuda")
               for s_ in (21, 22, 23))
    qs, ks, vs = zigzag_shares(q, P), zigzag_shares(k, P), zigzag_shares(v, P)
    kc, vc = [x.cpu() for x in ks], [x.cpu() for x in vs]
    for r in range(P):
        o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=True)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle.zigzag_ring_rank(qs[r].cpu(), kc, vc, r, causal=True)
        check_fp32(o.cpu(), ref_o, f"zigzag fp32 r{r}")
        assert oracle.max_abs_err(lse.cpu(), ref_lse) <= 1e-4


def test_zigzag_long_context_ranks_0_and_7():
    """L = 131072, H = 64, P = 8 zigzag shares (chunks of 8192 rows), ranks 0
    and 7, in the launch configuration the bench times: sampled rows of both
    chunks against the plain definition at their global positions."""
    w = W.LONG_ZIGZAG
    P, c = w.P, w.S_padded // (2 * w.P)
    say(w.name, "generate on device")
    q, k, v = W.make_qkv(w, device="cuda")
    ks, vs = zigzag_shares(k, P), zigzag_shares(v, P)
    heads = list(range(0, w.H, 8))
    for r in w.ranks:
        q_r = zigzag_shares(q, P)[r]
        say(w.name, "rank", r)
        o, lse = ra.zigzag_attn_fwd(q_r, ks, vs, r, causal=True)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all()
        for half, chunk in enumerate(oracle.zigzag_chunks(P, r)):
            rows = np.unique(np.concatenate([np.arange(0, c, 512), np.arange(0, 4),
                                             np.arange(c - 4, c), np.arange(126, 130)]))
            q_c = q[:, chunk * c:(chunk + 1) * c]
            klim = (chunk + 1) * c
            kc, vc = k[:, :klim].cpu(), v[:, :klim].cpu()
            ref_o, ref_l = [], []
            for h in heads:
                o_h, l_h, _, _ = oracle.attention(q_c[:, :, h:h + 1].cpu(), kc[:, :, h:h + 1],
                                                  vc[:, :, h:h + 1], causal=True,
                                                  q_pos0=chunk * c, k_pos0=0, rows=rows)
                ref_o.append(o_h)
                ref_l.append(l_h)
            got = o[:, half * c + rows][:, :, heads].cpu()
            check_bf16(got, np.concatenate(ref_o, 2), f"{w.name} r{r} chunk {chunk}")
            check_lse(lse[:, half * c + rows][:, :, heads].cpu(), np.concatenate(ref_l, 2),
                      f"{w.name} r{r} chunk {chunk}")


# ------------------------------------------------------------ grouped-query attention
@pytest.mark.parametrize("Hkv", [1, 2, 8])
def test_gqa_ring_all_ranks(variant, Hkv):
    """K/V with H_kv of H = 8 heads (multi-query, grouped, plain), B = 2,
    causal: every rank against the plain definition with query head h
    reading K/V head h / (H / H_kv)."""
    B, S, H, D, P = 2, 2048, 8, 128, 4
    Sb = S // P
    q = W.random_tensor((B, S, H, D), seed=51, device="cuda")
    k = W.random_tensor((B, S, Hkv, D), seed=52, device="cuda")
    v = W.random_tensor((B, S, Hkv, D), seed=53, device="cuda")
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    ke, ve = oracle.gqa_expand(k.cpu(), H), oracle.gqa_expand(v.cpu(), H)
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=True)
        torch.cuda.synchronize()
        ref_o, ref_lse, _, _ = oracle.attention(q_r.cpu(), ke[:, :(r + 1) * Sb], ve[:, :(r + 1) * Sb],
                                                causal=True, q_pos0=r * Sb, k_pos0=0)
        check_bf16(o.cpu(), ref_o, f"gqa Hkv={Hkv} r{r}")
        check_lse(lse.cpu(), ref_lse)


def test_gqa_fp32_and_bad_heads():
    """The fp32 kernel reads the grouped K/V heads too; a K/V head count that
    does not divide H is refused (ValueError) before any launch."""
    B, S, H, D, P, Hkv = 1, 512, 4, 64, 2, 2
    Sb = S // P
    q = W.random_tensor((B, S, H, D), dtype=torch.float32, seed=61, device="cuda")
    k = W.random_tensor((B, S, Hkv, D), dtype=torch.float32, seed=62, device="cuda")
    v = W.random_tensor((B, S, Hkv, D), dtype=torch.float32, seed=63, device="cuda")
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    ke, ve = oracle.gqa_expand(k.cpu(), H), oracle.gqa_expand(v.cpu(), H)
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        o, _ = ra.ring_attn_fwd(q_r, kb, vb, r, causal=False)
        torch.cuda.synchronize()
        ref_o, _, _, _ = oracle.attention(q_r.cpu(), ke, ve, causal=False, q_pos0=r * Sb)
        check_fp32(o.cpu(), ref_o, f"gqa fp32 r{r}")
    k3 = [x[:, :, :1].repeat(1, 1, 3, 1).contiguous() for x in kb]
    with pytest.raises(ValueError):
        ra.ring_attn_fwd(q[:, :Sb].contiguous(), k3, k3, 0)


# ------------------------------------------------------------ packed samples
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_all_ranks(variant, causal):
    """Packed samples (boundaries across the rank shares, a tail outside
    every sample): every rank against the oracle's same-sample attention;
    rows outside every sample are left untouched."""
    S, H, D, P = 2048, 4, 128, 4
    Sb = S // P
    cu = [0, 300, 1000, 1148, 1900]
    q, k, v = (W.random_tensor((1, S, H, D), seed=s_, device="cuda") for s_ in (71, 72, 73))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        o, lse = ra.ring_attn_fwd_varlen(q_r, kb, vb, r, cu, causal=causal)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle.packed_attention(qc[:, r * Sb:(r + 1) * Sb], kc, vc, cu,
                                                 causal=causal, q_pos0=r * Sb)
        inside = np.flatnonzero(r * Sb + np.arange(Sb) < cu[-1])
        outside = np.flatnonzero(r * Sb + np.arange(Sb) >= cu[-1])
        if len(inside):
            check_bf16(o.cpu()[:, inside], ref_o[:, inside], f"varlen causal={causal} r{r}")
            check_lse(lse.cpu()[:, inside], ref_lse[:, inside])
        if len(outside):
            assert not o[:, outside].any()
            assert torch.isneginf(lse[:, outside]).all()


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_many_samples_one_launch(causal):
    """The bf16 samples of a share go to one launch, eight at a time, and a
    sample that spans more than eight visited blocks takes a launch of its
    own: P = 16 shares of 256 rows, 44 short samples (up to 11 meeting one
    share, some across two shares) over the first 1100 rows, then one sample
    over the remaining 2996 rows (up to 12 visited blocks for the last
    ranks), every rank against the oracle's same-sample attention."""
    S, H, D, P = 4096, 2, 64, 16
    Sb = S // P
    cu = [0] + [37 + 25 * i for i in range(43)] + [1100, S]
    q, k, v = (W.random_tensor((1, S, H, D), seed=s_, device="cuda") for s_ in (91, 92, 93))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        say("varlen many samples", causal, "rank", r)
        o, lse = ra.ring_attn_fwd_varlen(q_r, kb, vb, r, cu, causal=causal)
        torch.cuda.synchronize()
        ref_o, ref_lse = oracle.packed_attention(qc[:, r * Sb:(r + 1) * Sb], kc, vc, cu,
                                                 causal=causal, q_pos0=r * Sb)
        check_bf16(o.cpu(), ref_o, f"varlen many causal={causal} r{r}")
        check_lse(lse.cpu(), ref_lse, f"varlen many causal={causal} r{r}")


def test_varlen_fp32_and_bad_tables():
    """fp32 through the fp32 kernel to 1e-5; boundaries that do not start at
    0, decrease or run past the sequence are refused before any launch."""
    S, H, D, P = 1024, 2, 64, 2
    Sb = S // P
    cu = [0, 100, 611, 1024]
    q, k, v = (W.random_tensor((1, S, H, D), dtype=torch.float32, seed=s_, device="cuda")
               for s_ in (81, 82, 83))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    for r in range(P):
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        o, _ = ra.ring_attn_fwd_varlen(q_r, kb, vb, r, cu, causal=True)
        torch.cuda.synchronize()
        ref_o, _ = oracle.packed_attention(q.cpu()[:, r * Sb:(r + 1) * Sb], k.cpu(), v.cpu(), cu,
                                           causal=True, q_pos0=r * Sb)
        check_fp32(o.cpu(), ref_o, f"varlen fp32 r{r}")
    q0 = q[:, :Sb].contiguous()
    for bad in ([5, 600, 1024], [0, 600, 500, 1024], [0, 600, 1100]):
        with pytest.raises(ValueError):
            ra.ring_attn_fwd_varlen(q0, kb, vb, 0, bad)


# ------------------------------------------------------------ ring backward
# Gradient tolerances (bf16 operands, fp32 accumulation): P and dS are
# rounded to bf16 (relative 2^-9) before their matrix products, as O's P is
# in the forward; against the fp64 oracle fed the same saved O and lse we
# require cos > 0.999, rel-L2 < 1e-2 and max_abs_err <= 1e-2 * max|ref|
# (the forward's absolute 1e-2 bound, scaled to the gradient's magnitude,
# which grows with the number of rows a block is summed over).
def check_grad(got, ref, what):
    c = oracle.compare(got, ref)
    scale = max(1.0, float(np.max(np.abs(ref))))
    say(what, {k: f"{v:.3e}" for k, v in c.items()}, f"max|ref| {scale:.3e}")
    assert np.all(np.isfinite(_f64(got)))
    assert c["max_abs_err"] <= 1e-2 * scale, (what, c)
    # cosine and relative L2 mean nothing for a gradient that is zero up to
    # rounding (one visible key: dS = P (dP - D) = 0 exactly)
    if float(np.max(np.abs(ref))) > 1e-6:
        assert c["cos"] > 0.999, (what, c)
        assert c["rel_l2"] < 1e-2, (what, c)


@pytest.mark.parametrize("D,causal,pad", [(128, True, 0), (128, False, 0), (64, True, 37)])
def test_ring_backward_all_ranks(D, causal, pad):
    """Every rank's backward (dq, and its dk/dv parts of the blocks it
    visits) against the oracle's ring backward fed the same saved O and
    lse; then the parts summed over all ranks (accumulated into the same
    buffers, as the ring returns them to the owners) against the
    full-sequence gradients of the plain definition."""
    B, S, H, P = 2, 1024, 3, 4
    Sb = S // P
    valid = S - pad
    q, k, v, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (31, 32, 33, 34))
    if pad:
        # padding rows of the inputs are zero; dO stays random there: the
        # padding queries are discarded and must not reach any gradient
        for x in (q, k, v):
            x[:, valid:] = 0
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    kc, vc = [x.cpu() for x in kb], [x.cpu() for x in vb]
    dk_all = [torch.zeros((B, Sb, H, D), dtype=torch.float32, device="cuda") for _ in range(P)]
    dv_all = [torch.zeros((B, Sb, H, D), dtype=torch.float32, device="cuda") for _ in range(P)]
    dq_all = []
    for r in range(P):
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
        o_r, lse_r = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid)
        say("ring bwd", D, causal, pad, "rank", r)
        dq, dk, dv = ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, r, causal=causal,
                                      valid_len=valid)
        ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, r, causal=causal, valid_len=valid,
                         dq=torch.zeros_like(dq), dk_blocks=dk_all, dv_blocks=dv_all)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.ring_attention_bwd_rank(q_r.cpu(), kc, vc, do_r.cpu(), r,
                                                    o_r=o_r.cpu(), lse_r=lse_r.cpu(),
                                                    causal=causal, valid_len=valid)
        check_grad(dq.cpu(), rq, f"dq r{r}")
        for j in range(P):
            if np.any(rk[j]):
                check_grad(dk[j].cpu(), rk[j], f"dk r{r} block {j}")
                check_grad(dv[j].cpu(), rv[j], f"dv r{r} block {j}")
            else:
                assert not dk[j].any() and not dv[j].any()
        dq_all.append(dq.cpu())
    fq, fk, fv = oracle.attention_grad(q.cpu(), k.cpu(), v.cpu(), do.cpu(), causal=causal,
                                       valid_len=valid)
    real = np.arange(valid)
    check_grad(torch.cat(dq_all, 1)[:, real], fq[:, real], "dq all ranks vs full")
    check_grad(torch.cat([x.cpu() for x in dk_all], 1)[:, real], fk[:, real], "dk owners vs full")
    check_grad(torch.cat([x.cpu() for x in dv_all], 1)[:, real], fv[:, real], "dv owners vs full")


@pytest.mark.parametrize("D,causal,pad", [(128, True, 0), (64, True, 37), (64, False, 0)])
def test_ring_backward_dq_waves(D, causal, pad):
    """The dQ kernel in 4- and 8-wave workgroups (RA_OPT_ATTN_WAVES forces
    either): every row's dq is formed by one wave in the same order both
    ways (shares this small never take the lockstep order), so the two are
    bit-identical, and both match the oracle.  320 rows per rank leave the
    last 8-wave workgroup with six empty waves."""
    B, H, P, Sb = 2, 3, 4, 320
    S = P * Sb
    valid = S - pad
    q, k, v, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (71, 72, 73, 74))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    kc, vc = [x.cpu() for x in kb], [x.cpu() for x in vb]
    for r in (1, P - 1):
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
        o_r, lse_r = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid)
        got = {}
        try:
            for wv in (4, 8):
                ra.set_attn_waves(wv)
                say("ring bwd dq waves", wv, D, causal, pad, "rank", r)
                got[wv] = ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, r, causal=causal,
                                           valid_len=valid)
                torch.cuda.synchronize()
        finally:
            ra.set_attn_waves(0)
        assert torch.equal(got[4][0], got[8][0])
        for j in range(P):
            assert torch.equal(got[4][1][j], got[8][1][j]) and torch.equal(got[4][2][j], got[8][2][j])
        rq, rk, rv = oracle.ring_attention_bwd_rank(q_r.cpu(), kc, vc, do_r.cpu(), r,
                                                    o_r=o_r.cpu(), lse_r=lse_r.cpu(),
                                                    causal=causal, valid_len=valid)
        check_grad(got[8][0].cpu(), rq, f"dq 8 waves r{r}")
        for j in range(P):
            if np.any(rk[j]):
                check_grad(got[8][1][j].cpu(), rk[j], f"dk r{r} block {j}")
                check_grad(got[8][2][j].cpu(), rv[j], f"dv r{r} block {j}")


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_block_backward_rounds(D, causal):
    """ra_block_attn_bwd one round at a time: a query shard of 200 rows
    (global rows 300..499) against four K/V blocks of uneven, ragged
    lengths (130, 170, 220, 180 keys; real length 610, the rest padding).
    Each block's dq, dk and dv terms against the oracle's gradients of that
    block from the same saved O and lse; the rounds' dq summed against the
    plain definition.  Causal: the last block lies after every query (SKIP)
    and must leave the buffers untouched."""
    B, H, Sq, q0, valid = 2, 3, 200, 300, 610
    bounds = [0, 130, 300, 520, 700]
    S = bounds[-1]
    qf, k, v, dof = (W.random_tensor((B, S, H, D), seed=s_) for s_ in (51, 52, 53, 54))
    q = qf[:, q0:q0 + Sq].contiguous()
    do = dof[:, q0:q0 + Sq].contiguous()
    of, lsef, _, _ = oracle.attention(q, k, v, causal=causal, q_pos0=q0, valid_len=valid)
    o = torch.from_numpy(of).to(torch.bfloat16)
    lse = torch.from_numpy(lsef).to(torch.float32)
    qg, dog, og, lg = (x.cuda() for x in (q, do, o, lse))
    dq_sum = torch.zeros((B, Sq, H, D), dtype=torch.float32, device="cuda")
    for a_, b_ in zip(bounds[:-1], bounds[1:]):
        kb, vb = k[:, a_:b_].contiguous(), v[:, a_:b_].contiguous()
        say("block bwd", D, causal, "keys", a_, b_)
        sentinel = 7.0
        dq = torch.full((B, Sq, H, D), sentinel, dtype=torch.float32, device="cuda")
        dk = torch.full(kb.shape, sentinel, dtype=torch.float32, device="cuda")
        dv = torch.full(kb.shape, sentinel, dtype=torch.float32, device="cuda")
        ra.block_attn_bwd(qg, kb.cuda(), vb.cuda(), og, dog, lg, q_pos0=q0, k_pos0=a_,
                          causal=causal, valid_len=valid, dq=dq, dk=dk, dv=dv)
        ra.block_attn_bwd(qg, kb.cuda(), vb.cuda(), og, dog, lg, q_pos0=q0, k_pos0=a_,
                          causal=causal, valid_len=valid, dq=dq_sum)
        torch.cuda.synchronize()
        if causal and a_ > q0 + Sq - 1:
            for t in (dq, dk, dv):
                assert bool((t == sentinel).all())
            continue
        rq, rk, rv = oracle.attention_grad_sampled(q, kb, vb, do, o, lse, q_rows=np.arange(Sq),
                                                   k_rows=np.arange(b_ - a_), causal=causal,
                                                   q_pos0=q0, k_pos0=a_, valid_len=valid)
        check_grad(dq.cpu() - sentinel, rq, f"dq keys {a_}..{b_}")
        check_grad(dk.cpu() - sentinel, rk, f"dk keys {a_}..{b_}")
        check_grad(dv.cpu() - sentinel, rv, f"dv keys {a_}..{b_}")
    fq, _, _ = oracle.attention_grad(q, k, v, do, causal=causal, q_pos0=q0, valid_len=valid)
    check_grad(dq_sum.cpu(), fq, "dq summed over the rounds vs the plain definition")


@pytest.mark.parametrize("D,causal,pad", [(128, True, 0), (64, True, 41), (128, False, 0)])
def test_zigzag_backward_all_ranks(D, causal, pad):
    """Zigzag ring backward (chunks of 192 rows: the last 128-key tile of
    every chunk is half full), B = 2: every rank's dq against the rows of the
    full-sequence gradient at its share's positions, and the dk/dv parts of
    all ranks accumulated into the share buffers against the full-sequence
    gradients at each share's positions (real rows; the padded case masks
    the last 41 keys)."""
    B, S, H, P = 2, 1536, 3, 4
    c = S // (2 * P)
    valid = S - pad
    q, k, v, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (71, 72, 73, 74))
    if pad:
        # padding rows of the inputs are zero; dO stays random there: the
        # padding queries are discarded and must not reach any gradient
        for x in (q, k, v):
            x[:, valid:] = 0
    qs, ks, vs, dos = (zigzag_shares(x, P) for x in (q, k, v, do))
    f32 = dict(dtype=torch.float32, device="cuda")
    dk_all = [torch.zeros(x.shape, **f32) for x in ks]
    dv_all = [torch.zeros(x.shape, **f32) for x in ks]
    fq, fk, fv = oracle.attention_grad(q.cpu(), k.cpu(), v.cpu(), do.cpu(), causal=causal,
                                       valid_len=valid)
    for r in range(P):
        say("zigzag bwd", D, causal, pad, "rank", r)
        o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=causal, valid_len=valid)
        dq, _, _ = ra.zigzag_attn_bwd(qs[r], ks, vs, o, dos[r], lse, r, causal=causal,
                                      valid_len=valid, dk_shares=dk_all, dv_shares=dv_all)
        torch.cuda.synchronize()
        pos = np.asarray(oracle.zigzag_positions(P, r, c))
        real = pos < valid
        check_grad(dq.cpu()[:, real], fq[:, pos[real]], f"zigzag dq r{r}")
    for j in range(P):
        pos = np.asarray(oracle.zigzag_positions(P, j, c))
        real = pos < valid
        check_grad(dk_all[j].cpu()[:, real], fk[:, pos[real]], f"zigzag dk share {j}")
        check_grad(dv_all[j].cpu()[:, real], fv[:, pos[real]], f"zigzag dv share {j}")


@pytest.mark.parametrize("Hkv,causal,pad", [(1, True, 0), (2, True, 37), (2, False, 0)])
def test_gqa_backward_all_ranks(Hkv, causal, pad):
    """Grouped-query ring backward (4 query heads on 1 or 2 K/V heads), B =
    2, every rank: dq against the full-sequence gradient, and the dK/dV parts
    of all ranks accumulated into the owners' buffers against the
    full-sequence gradients of the expanded K/V summed over each group."""
    B, S, H, D, P = 2, 1024, 4, 128, 4
    Sb, valid, G = S // P, S - pad, H // Hkv
    q, do = (W.random_tensor((B, S, H, D), seed=s_, device="cuda") for s_ in (81, 84))
    k, v = (W.random_tensor((B, S, Hkv, D), seed=s_, device="cuda") for s_ in (82, 83))
    if pad:
        # padding rows of the inputs are zero; dO stays random there: the
        # padding queries are discarded and must not reach any gradient
        for x in (q, k, v):
            x[:, valid:] = 0
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    f32 = dict(dtype=torch.float32, device="cuda")
    dk_all = [torch.zeros((B, Sb, Hkv, D), **f32) for _ in range(P)]
    dv_all = [torch.zeros((B, Sb, Hkv, D), **f32) for _ in range(P)]
    fq, fk, fv = oracle.attention_grad(q.cpu(), oracle.gqa_expand(k.cpu(), H),
                                       oracle.gqa_expand(v.cpu(), H), do.cpu(), causal=causal,
                                       valid_len=valid)
    fk = fk.reshape(B, S, Hkv, G, D).sum(axis=3)
    fv = fv.reshape(B, S, Hkv, G, D).sum(axis=3)
    real = np.arange(valid)
    dqs = []
    for r in range(P):
        say("gqa bwd", Hkv, causal, pad, "rank", r)
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
        o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid)
        dq, _, _ = ra.ring_attn_bwd(q_r, kb, vb, o, do_r, lse, r, causal=causal, valid_len=valid,
                                    dk_blocks=dk_all, dv_blocks=dv_all)
        torch.cuda.synchronize()
        dqs.append(dq.cpu())
    check_grad(torch.cat(dqs, 1)[:, real], fq[:, real], "gqa dq all ranks")
    check_grad(torch.cat([x.cpu() for x in dk_all], 1)[:, real], fk[:, real], "gqa dk owners")
    check_grad(torch.cat([x.cpu() for x in dv_all], 1)[:, real], fv[:, real], "gqa dv owners")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_backward_all_ranks(causal):
    """Backward over packed samples (boundaries across the rank shares and
    inside blocks, a tail outside every sample), every rank: dq, and the
    dK/dV parts of all ranks accumulated into the owners' buffers, against
    the plain gradients of each sample on its own; rows outside every sample
    stay zero."""
    S, H, D, P = 2048, 3, 128, 4
    Sb = S // P
    cu = [0, 300, 1000, 1148, 1900]
    q, k, v, do = (W.random_tensor((1, S, H, D), seed=s_, device="cuda") for s_ in (91, 92, 93, 94))
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    f32 = dict(dtype=torch.float32, device="cuda")
    dk_all = [torch.zeros((1, Sb, H, D), **f32) for _ in range(P)]
    dv_all = [torch.zeros((1, Sb, H, D), **f32) for _ in range(P)]
    fq, fk, fv = (np.zeros((1, S, H, D)) for _ in range(3))
    qc, kc, vc, dc = q.cpu(), k.cpu(), v.cpu(), do.cpu()
    for s0, s1 in zip(cu[:-1], cu[1:]):
        g = oracle.attention_grad(qc[:, s0:s1], kc[:, s0:s1], vc[:, s0:s1], dc[:, s0:s1],
                                  causal=causal)
        fq[:, s0:s1], fk[:, s0:s1], fv[:, s0:s1] = g
    dqs = []
    for r in range(P):
        say("varlen bwd", causal, "rank", r)
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
        o, lse = ra.ring_attn_fwd_varlen(q_r, kb, vb, r, cu, causal=causal)
        dq, _, _ = ra.ring_attn_bwd_varlen(q_r, kb, vb, o, do_r, lse, r, cu, causal=causal,
                                           dk_blocks=dk_all, dv_blocks=dv_all)
        torch.cuda.synchronize()
        dqs.append(dq.cpu())
    real = np.arange(cu[-1])
    check_grad(torch.cat(dqs, 1)[:, real], fq[:, real], "varlen dq all ranks")
    check_grad(torch.cat([x.cpu() for x in dk_all], 1)[:, real], fk[:, real], "varlen dk owners")
    check_grad(torch.cat([x.cpu() for x in dv_all], 1)[:, real], fv[:, real], "varlen dv owners")
    tail = np.arange(cu[-1], S)
    for x in (torch.cat(dqs, 1), torch.cat([y.cpu() for y in dk_all], 1),
              torch.cat([y.cpu() for y in dv_all], 1)):
        assert not x[:, tail].any()


# ------------------------------------------------------------ fp32 backward
def check_grad_fp32(got, ref, what):
    """fp32 inputs: the fp32 tier (1e-5 absolute, fused-operator precision
    page §3.4), relative to the gradient's scale where it exceeds 1."""
    c = oracle.compare(got, ref)
    scale = max(1.0, float(np.max(np.abs(ref))))
    say(what, {k: f"{v:.3e}" for k, v in c.items()}, f"max|ref| {scale:.3e}")
    assert np.all(np.isfinite(_f64(got)))
    assert c["max_abs_err"] <= FP32_ATOL * scale, (what, c)


def f32_tensors(shapes_seeds, valid=None):
    out = [W.random_tensor(shp, dtype=torch.float32, seed=s_, device="cuda")
           for shp, s_ in shapes_seeds]
    return out


@pytest.mark.parametrize("D,causal,pad,Hkv", [(64, False, 0, 2), (128, True, 37, 2),
                                              (64, True, 0, 1)])
def test_fp32_ring_backward(D, causal, pad, Hkv):
    """fp32 ring backward (grouped-query when Hkv < H), B = 2, every rank,
    96 rows per rank (ragged 32-row tiles): dq of all ranks and the dK/dV
    parts accumulated into the owners' buffers against the full-sequence
    gradients of the plain definition at the fp32 tier."""
    B, H, P, Sb = 2, 2, 4, 96
    S, G = P * Sb, H // Hkv
    valid = S - pad
    q, do = f32_tensors([((B, S, H, D), 101), ((B, S, H, D), 104)])
    k, v = f32_tensors([((B, S, Hkv, D), 102), ((B, S, Hkv, D), 103)])
    if pad:
        # padding rows of the inputs are zero; dO stays random there
        for x in (q, k, v):
            x[:, valid:] = 0
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    f32 = dict(dtype=torch.float32, device="cuda")
    dk_all = [torch.zeros((B, Sb, Hkv, D), **f32) for _ in range(P)]
    dv_all = [torch.zeros((B, Sb, Hkv, D), **f32) for _ in range(P)]
    fq, fk, fv = oracle.attention_grad(q.cpu(), oracle.gqa_expand(k.cpu(), H),
                                       oracle.gqa_expand(v.cpu(), H), do.cpu(), causal=causal,
                                       valid_len=valid)
    fk = fk.reshape(B, S, Hkv, G, D).sum(axis=3)
    fv = fv.reshape(B, S, Hkv, G, D).sum(axis=3)
    dqs = []
    for r in range(P):
        say("fp32 ring bwd", D, causal, pad, Hkv, "rank", r)
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
        o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=causal, valid_len=valid)
        dq, _, _ = ra.ring_attn_bwd(q_r, kb, vb, o, do_r, lse, r, causal=causal, valid_len=valid,
                                    dk_blocks=dk_all, dv_blocks=dv_all)
        torch.cuda.synchronize()
        dqs.append(dq.cpu())
    real = np.arange(valid)
    check_grad_fp32(torch.cat(dqs, 1)[:, real], fq[:, real], "fp32 dq all ranks")
    check_grad_fp32(torch.cat([x.cpu() for x in dk_all], 1)[:, real], fk[:, real], "fp32 dk owners")
    check_grad_fp32(torch.cat([x.cpu() for x in dv_all], 1)[:, real], fv[:, real], "fp32 dv owners")
    pad_rows = np.arange(valid, S)
    assert not torch.cat(dqs, 1)[:, pad_rows].any()


def test_fp32_zigzag_block_and_varlen_backward():
    """The other fp32 backward forms against the plain definition at the
    fp32 tier: zigzag shares (chunks of 128 rows, causal, 29 padding
    tokens), one round at a time (ra_block_attn_bwd over every block, the
    rank's lse from the whole forward), and packed samples."""
    B, H, D, P = 1, 2, 64, 4
    S = 1024
    c = S // (2 * P)
    valid = S - 29
    q, k, v, do = f32_tensors([((B, S, H, D), s_) for s_ in (111, 112, 113, 114)])
    for x in (q, k, v):
        x[:, valid:] = 0
    fq, fk, fv = oracle.attention_grad(q.cpu(), k.cpu(), v.cpu(), do.cpu(), causal=True,
                                       valid_len=valid)
    qs, ks, vs, dos = (zigzag_shares(x, P) for x in (q, k, v, do))
    f32 = dict(dtype=torch.float32, device="cuda")
    dk_all = [torch.zeros(x.shape, **f32) for x in ks]
    dv_all = [torch.zeros(x.shape, **f32) for x in ks]
    for r in range(P):
        say("fp32 zigzag bwd rank", r)
        o, lse = ra.zigzag_attn_fwd(qs[r], ks, vs, r, causal=True, valid_len=valid)
        dq, _, _ = ra.zigzag_attn_bwd(qs[r], ks, vs, o, dos[r], lse, r, causal=True,
                                      valid_len=valid, dk_shares=dk_all, dv_shares=dv_all)
        torch.cuda.synchronize()
        pos = np.asarray(oracle.zigzag_positions(P, r, c))
        real = pos < valid
        check_grad_fp32(dq.cpu()[:, real], fq[:, pos[real]], f"fp32 zigzag dq r{r}")
    for j in range(P):
        pos = np.asarray(oracle.zigzag_positions(P, j, c))
        real = pos < valid
        check_grad_fp32(dk_all[j].cpu()[:, real], fk[:, pos[real]], f"fp32 zigzag dk share {j}")
        check_grad_fp32(dv_all[j].cpu()[:, real], fv[:, pos[real]], f"fp32 zigzag dv share {j}")

    # one round at a time: rank 2 of a contiguous P = 4 ring (blocks 2, 1, 0)
    Sb, r = S // P, 2
    sl = slice(r * Sb, (r + 1) * Sb)
    q_r, do_r = q[:, sl].contiguous(), do[:, sl].contiguous()
    kb, vb = blocks_of(k, P), blocks_of(v, P)
    o, lse = ra.ring_attn_fwd(q_r, kb, vb, r, causal=True, valid_len=valid)
    dq = torch.zeros(q_r.shape, **f32)
    for j in (2, 1, 0):
        say("fp32 block bwd block", j)
        _, dk, dv = ra.block_attn_bwd(q_r, kb[j], vb[j], o, do_r, lse, q_pos0=r * Sb,
                                      k_pos0=j * Sb, causal=True, valid_len=valid, dq=dq)
        torch.cuda.synchronize()
        # block j's keys get the terms of rank r's queries only
        rq, rk, rv = oracle.ring_attention_bwd_rank(q_r.cpu(), [x.cpu() for x in kb],
                                                    [x.cpu() for x in vb], do_r.cpu(), r,
                                                    o_r=o.cpu(), lse_r=lse.cpu(), causal=True,
                                                    valid_len=valid)
        check_grad_fp32(dk.cpu(), rk[j], f"fp32 block dk {j}")
        check_grad_fp32(dv.cpu(), rv[j], f"fp32 block dv {j}")
    check_grad_fp32(dq.cpu(), rq, "fp32 block dq (three rounds)")

    # packed samples
    cu = [0, 300, 700, 1000]
    q1, k1, v1, do1 = (x[:1] for x in (q, k, v, do))
    kb1, vb1 = blocks_of(k1, P), blocks_of(v1, P)
    dk_p = [torch.zeros((1, Sb, H, D), **f32) for _ in range(P)]
    dv_p = [torch.zeros((1, Sb, H, D), **f32) for _ in range(P)]
    gq, gk, gv = (np.zeros((1, S, H, D)) for _ in range(3))
    qc, kc, vc, dc = q1.cpu(), k1.cpu(), v1.cpu(), do1.cpu()
    for s0, s1 in zip(cu[:-1], cu[1:]):
        g = oracle.attention_grad(qc[:, s0:s1], kc[:, s0:s1], vc[:, s0:s1], dc[:, s0:s1],
                                  causal=True)
        gq[:, s0:s1], gk[:, s0:s1], gv[:, s0:s1] = g
    dqs = []
    for r in range(P):
        say("fp32 varlen bwd rank", r)
        sl = slice(r * Sb, (r + 1) * Sb)
        q_r, do_r = q1[:, sl].contiguous(), do1[:, sl].contiguous()
        o, lse = ra.ring_attn_fwd_varlen(q_r, kb1, vb1, r, cu, causal=True)
        dq, _, _ = ra.ring_attn_bwd_varlen(q_r, kb1, vb1, o, do_r, lse, r, cu, causal=True,
                                           dk_blocks=dk_p, dv_blocks=dv_p)
        torch.cuda.synchronize()
        dqs.append(dq.cpu())
    real = np.arange(cu[-1])
    check_grad_fp32(torch.cat(dqs, 1)[:, real], gq[:, real], "fp32 varlen dq")
    check_grad_fp32(torch.cat([x.cpu() for x in dk_p], 1)[:, real], gk[:, real], "fp32 varlen dk")
    check_grad_fp32(torch.cat([x.cpu() for x in dv_p], 1)[:, real], gv[:, real], "fp32 varlen dv")


def test_random_shapes_forward_and_backward():
    """Seeded random small shares (B, P, rows per rank from 1 to 300, heads
    and grouped K/V heads, D, causal, padding, rank): the ring forward (the
    binding's default, split or not) against the oracle's recurrence, and the
    ring backward against the oracle's ring backward fed the same saved O and
    lse (grouped K/V: the oracle on expanded blocks, parts summed per
    group)."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        B = int(rng.integers(1, 3))
        P = int(rng.choice([1, 2, 3, 5]))
        Sb = int(rng.integers(1, 301))
        H = int(rng.choice([1, 2, 3, 4]))
        Hkv = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        r = int(rng.integers(0, P))
        valid = P * Sb - int(rng.integers(0, Sb))
        say("random case", case, dict(B=B, P=P, Sb=Sb, H=H, Hkv=Hkv, D=D, causal=causal, r=r,
                                      valid=valid))
        S = P * Sb
        seed = 1000 + 10 * case
        q = W.random_tensor((B, S, H, D), seed=seed)
        k = W.random_tensor((B, S, Hkv, D), seed=seed + 1)
        v = W.random_tensor((B, S, Hkv, D), seed=seed + 2)
        q_r = q[:, r * Sb:(r + 1) * Sb].contiguous()
        do_r = W.random_tensor(q_r.shape, seed=seed + 3)
        kb, vb = blocks_of(k, P), blocks_of(v, P)
        kg, vg = [x.cuda() for x in kb], [x.cuda() for x in vb]
        o, lse = ra.ring_attn_fwd(q_r.cuda(), kg, vg, r, causal=causal, valid_len=valid)
        dq, dk, dv = ra.ring_attn_bwd(q_r.cuda(), kg, vg, o, do_r.cuda(), lse, r, causal=causal,
                                      valid_len=valid)
        torch.cuda.synchronize()
        ke = [oracle.gqa_expand(x, H) for x in kb]
        ve = [oracle.gqa_expand(x, H) for x in vb]
        ref_o, ref_lse = oracle.ring_attention_rank(q_r, ke, ve, r, causal=causal, valid_len=valid)
        rows = np.arange(max(0, min(Sb, valid - r * Sb)))
        if len(rows):
            check_bf16(o.cpu()[:, rows], ref_o[:, rows], f"random {case} O")
            check_lse(lse.cpu()[:, rows], ref_lse[:, rows])
        rq, rk, rv = oracle.ring_attention_bwd_rank(q_r, ke, ve, do_r, r, o_r=o.cpu(),
                                                    lse_r=lse.cpu(), causal=causal,
                                                    valid_len=valid)
        check_grad(dq.cpu(), rq, f"random {case} dq")
        G = H // Hkv
        for j in range(P):
            gk = rk[j].reshape(B, Sb, Hkv, G, D).sum(axis=3)
            gv = rv[j].reshape(B, Sb, Hkv, G, D).sum(axis=3)
            if np.any(gk) or np.any(gv):
                check_grad(dk[j].cpu(), gk, f"random {case} dk {j}")
                check_grad(dv[j].cpu(), gv, f"random {case} dv {j}")
            else:
                assert not dk[j].any() and not dv[j].any()


def test_ring_backward_long_context_rank3():
    """L = 131072, H = 64, P = 8, rank 3 (the bench share): dq on sampled
    rows and dk / dv on sampled keys of the diagonal and the first block,
    against the oracle evaluated from the same saved O and lse."""
    w = W.LONG_CAUSAL
    r, Sb = 3, w.block_len
    say(w.name, "backward: generate on device")
    q, k, v = W.make_qkv(w, device="cuda")
    kb = [k[:, j * Sb:(j + 1) * Sb] for j in range(w.P)]
    vb = [v[:, j * Sb:(j + 1) * Sb] for j in range(w.P)]
    q_r = q[:, r * Sb:(r + 1) * Sb]
    do_r = W.random_tensor(q_r.shape, seed=41, device="cuda")
    o_r, lse_r = ra.ring_attn_fwd(q_r, kb, vb, r, causal=True)
    say(w.name, "backward rank 3")
    dq, dk, dv = ra.ring_attn_bwd(q_r, kb, vb, o_r, do_r, lse_r, r, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all()
    for j in range(r + 1, w.P):
        assert not dk[j].any() and not dv[j].any()
    # query rows at a stride co-prime to the tiles, keys likewise
    q_rows = np.unique(np.concatenate([np.arange(0, Sb, 1021), [1, 63, 64, 127, Sb - 1]]))
    k_local = np.unique(np.concatenate([[0, 1, 63, 64, 5000, Sb - 2, Sb - 1],
                                        np.arange(37, Sb, 1531)]))
    heads = [0, 21, 42, 63]
    kc = k[:, :(r + 1) * Sb].cpu()
    vc = v[:, :(r + 1) * Sb].cpu()
    qc, dc, oc, lc = q_r.cpu(), do_r.cpu(), o_r.cpu(), lse_r.cpu()
    for j in (0, r):
        for h in heads:
            hs = slice(h, h + 1)
            sq, sk, sv = oracle.attention_grad_sampled(
                qc[:, :, hs], kc[:, :, hs], vc[:, :, hs], dc[:, :, hs], oc[:, :, hs], lc[:, :, hs],
                q_rows=q_rows, k_rows=j * Sb + k_local, causal=True, q_pos0=r * Sb, k_pos0=0)
            check_grad(dk[j][:, k_local, hs].cpu(), sk, f"dk block {j} head {h}")
            check_grad(dv[j][:, k_local, hs].cpu(), sv, f"dv block {j} head {h}")
            if j == r:
                check_grad(dq[:, q_rows, hs].cpu(), sq, f"dq head {h}")


# ------------------------------------------------------------ merge kernel
def test_ring_merge_against_oracle():
    g = torch.Generator().manual_seed(5)
    B, Sq, H, D = 2, 37, 3, 64
    o1 = torch.randn(B, Sq, H, D, generator=g)
    o2 = torch.randn(B, Sq, H, D, generator=g)
    l1 = torch.randn(B, Sq, H, generator=g) * 4
    l2 = torch.randn(B, Sq, H, generator=g) * 4
    l1[0, :5] = -math.inf                      # empty partials on either side
    l2[0, 3:8] = -math.inf
    o1[0, :5] = 0
    o2[0, 3:8] = 0
    ref_o, ref_l = oracle.lse_combine(o1, l1, o2, l2)
    oa, la = o1.cuda(), l1.cuda()
    fin = torch.empty(B, Sq, H, D, dtype=torch.bfloat16, device="cuda")
    say("merge")
    ra.ring_merge(oa, la, o2.cuda(), l2.cuda(), out_final=fin)
    torch.cuda.synchronize()
    assert torch.isfinite(oa).all()
    check_fp32(oa.cpu(), ref_o, "merge o", atol=2e-6)
    lg = la.cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
    fin_ref = torch.from_numpy(ref_o).float().to(torch.bfloat16)
    assert torch.equal(fin.cpu().view(torch.int16), fin_ref.view(torch.int16)) or \
        (fin.cpu().float() - fin_ref.float()).abs().max().item() <= 2 ** -7
    m = np.isfinite(ref_l)
    np.testing.assert_allclose(lg[m], ref_l[m], atol=2e-6)


# ------------------------------------------------------------ edge cases
def test_edge_cases_fp32():
    g = torch.Generator().manual_seed(9)
    mk = lambda *s: torch.randn(*s, generator=g)
    # one query, one key; ragged tiles; non-default scale
    for (B, Sq, Sk, H, D) in [(1, 1, 1, 1, 64), (2, 130, 67, 3, 64), (1, 33, 200, 2, 128)]:
        q, k, v = mk(B, Sq, H, D), mk(B, Sk, H, D), mk(B, Sk, H, D)
        for causal, qp, kp in [(False, 0, 0), (True, 100, 0), (True, 0, 0)]:
            say("edge", (B, Sq, Sk, H, D), causal, qp, kp)
            o, lse, m, l = ra.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=0.3,
                                             q_pos0=qp, k_pos0=kp, causal=causal)
            torch.cuda.synchronize()
            ro, rl, rm, rl2 = oracle.attention(q, k, v, scale=0.3, q_pos0=qp, k_pos0=kp,
                                               causal=causal)
            check_fp32(o.cpu(), ro, "edge o")
            lg = lse.cpu().numpy()
            assert np.array_equal(np.isneginf(lg), np.isneginf(rl))   # unseen rows
            fin = np.isfinite(rl)
            np.testing.assert_allclose(lg[fin], rl[fin], atol=1e-5)
            assert np.all(o.cpu().numpy()[~fin] == 0)


def test_edge_empty_inputs():
    say("edge empty")
    z = torch.zeros(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    q = torch.randn(1, 5, 2, 64, device="cuda").to(torch.bfloat16)
    o, lse, m, l = ra.block_attn_fwd(q, z, z)              # no keys at all
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse)) and torch.all(l == 0)
    o, lse, _, _ = ra.block_attn_fwd(z, q, q)              # no queries
    assert o.numel() == 0
    e = torch.zeros(2, 0, 0, 4, 64, dtype=torch.bfloat16, device="cuda")
    assert ra.seq2head(e).shape == (2, 0, 0, 2, 64)
    with pytest.raises(ValueError):
        ra.seq2head(torch.zeros(3, 1, 2, 4, 8, dtype=torch.bfloat16, device="cuda"))


def test_stability_large_scores():
    """Tutorial §09: large scores stay finite.  K' = K + w adds q_i.w to every
    score of row i (a per-row shift of ~1e3, which a naive exp overflows);
    the GPU result matches the oracle on the same shifted inputs."""
    g = torch.Generator().manual_seed(4)
    B, S, H, D = 1, 256, 2, 64
    q, k, v = (torch.randn(B, S, H, D, generator=g) for _ in range(3))
    wv = torch.zeros(D)
    wv[0] = 8000.0
    k2 = k + wv
    say("stability")
    o, lse = ra.ring_attn_fwd(q.cuda(), [k2.cuda()], [v.cuda()], 0)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    ref, _, _, _ = oracle.attention(q, k2, v)
    s = oracle.scores(q, k2, 1 / math.sqrt(D))
    assert np.abs(s).max() > 1000          # the shift really is large
    # fp32 scores of magnitude ~1e3 carry ~1e-4 absolute rounding, which the
    # exponent turns into relative weight errors of that size
    check_fp32(o.cpu(), ref, "stability", atol=2e-3)


def test_edge_cases_bf16(variant):
    """bf16 through both kernels: ragged query and key tiles, causal offsets
    (including rows that see no key), padding, non-default scale."""
    g = torch.Generator().manual_seed(19)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    for (B, Sq, Sk, H, D) in [(1, 1, 1, 1, 64), (2, 300, 67, 3, 64), (1, 33, 200, 2, 128),
                              (1, 520, 777, 2, 128)]:
        q, k, v = mk(B, Sq, H, D), mk(B, Sk, H, D), mk(B, Sk, H, D)
        for causal, qp, kp, vl in [(False, 0, 0, -1), (True, 100, 0, -1), (True, 0, 50, -1),
                                   (True, 300, 0, 250), (False, 0, 0, 40)]:
            say("edge bf16", variant, (B, Sq, Sk, H, D), causal, qp, kp, vl)
            o, lse, m, l = ra.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=0.11,
                                             q_pos0=qp, k_pos0=kp, causal=causal,
                                             valid_len=vl)
            torch.cuda.synchronize()
            ro, rl, rm, _ = oracle.attention(q, k, v, scale=0.11, q_pos0=qp, k_pos0=kp,
                                             causal=causal, valid_len=None if vl < 0 else vl)
            og = o.cpu().numpy()
            assert np.all(np.isfinite(og))
            assert oracle.max_abs_err(og, ro) <= BF16_ATOL, (variant, causal, qp, kp)
            if np.abs(ro).sum() > 0:
                assert oracle.cosine(og, ro) > BF16_COS
            lg = lse.cpu().numpy()
            assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
            fin = np.isfinite(rl)
            check_lse(lg[fin], rl[fin])
            assert np.all(og[~fin] == 0)


def test_eight_wave_loop_exits():
    """The 8-wave kernel runs four pipeline steps per loop iteration (its
    buffer indices are constants): one 256-row workgroup per head over 1 to
    9 key tiles and a ragged tenth, so the sequence ends after each of the
    four steps, with and without the exact row max, causal and not, at
    D = 128 and 64, against the oracle."""
    g = torch.Generator().manual_seed(23)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    ra.set_attn_waves(8)
    try:
        for D in (128, 64):
            q = mk(1, 256, 2, D)
            for Sk in [64 * n for n in range(1, 10)] + [64 * 9 + 17]:
                k, v = mk(1, Sk, 2, D), mk(1, Sk, 2, D)
                for causal, qp in [(False, 0), (True, max(0, Sk - 200))]:
                    for want_ml in (False, True):
                        say("8-wave loop exits", D, Sk, causal, want_ml)
                        o, lse, _, _ = ra.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), q_pos0=qp,
                                                         causal=causal, want_ml=want_ml)
                        torch.cuda.synchronize()
                        ro, rl, _, _ = oracle.attention(q, k, v, q_pos0=qp, causal=causal)
                        og = o.cpu().numpy()
                        assert oracle.max_abs_err(og, ro) <= BF16_ATOL, (D, Sk, causal, want_ml)
                        fin = np.isfinite(rl)
                        assert np.array_equal(np.isneginf(lse.cpu().numpy()), np.isneginf(rl))
                        check_lse(lse.cpu().numpy()[fin], rl[fin])
                        assert np.all(og[~fin] == 0)
    finally:
        ra.set_attn_waves(0)


# ------------------------------------------------------------ permutations
@pytest.mark.parametrize("P,B,S,H,D,dtype", [
    (8, 1, 16384, 32, 128, torch.int16),      # the Ulysses workload's shape (1 KiB runs)
    (2, 1, 64, 16, 128, torch.int16),         # 2 KiB runs: two pieces per run
    (4, 2, 256, 4, 128, torch.int16),         # 256-byte runs: four runs per piece
    (2, 1, 8, 2, 24, torch.int16),            # 48-byte runs: 16-byte path per unit
    (4, 2, 64, 8, 3, torch.int16),            # run of 6 bytes: element path
    (2, 3, 10, 4, 5, torch.int8),
    (4, 1, 32, 4, 16, torch.int32),
    (3, 1, 12, 3, 2, torch.int64),
])
def test_permutations_bit_exact(P, B, S, H, D, dtype):
    say("permute", (P, B, S, H, D, dtype))
    if dtype == torch.int16:
        x = W.random_bits16((P, B, S // P, H, D), seed=P + S)
    else:
        info = torch.iinfo(dtype)
        x = torch.randint(info.min, info.max, (P, B, S // P, H, D),
                          generator=torch.Generator().manual_seed(3), dtype=dtype)
    xg = x.cuda()
    hx = ra.seq2head(xg)
    back = ra.head2seq(hx)
    torch.cuda.synchronize()
    assert np.array_equal(hx.cpu().numpy(), oracle.seq2head(x.numpy()))
    assert torch.equal(back.cpu(), x)
    if P * B * S * H * D <= 4096:
        assert np.array_equal(hx.cpu().numpy(), oracle.seq2head_loops(x.numpy()))
