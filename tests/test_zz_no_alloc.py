"""The allocation-free split ring (ra_ring_attn_fwd_split_noalloc) against
the split ring with a caller workspace (ra_ring_attn_fwd_split), through the
C ABI: the same kernels run on the same plan, so the outputs must agree bit
for bit, and both must meet the bf16 bar against the oracle (max_abs_err
<= 1e-2, cos > 0.999, juejin post §二/§三).  Two calls in a row, the second
on a smaller share, so that the second reads scratch the first left behind;
and a plan too large for the fixed scratch is refused before any launch.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_ulysses_sequence_amd")


def _share(B, S, H, D, P, rank, causal, seed):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(3))
    Sb = S // P
    kb = [k[:, j * Sb:(j + 1) * Sb].contiguous().cuda() for j in range(P)]
    vb = [v[:, j * Sb:(j + 1) * Sb].contiguous().cuda() for j in range(P)]
    q_r = q[:, rank * Sb:(rank + 1) * Sb].contiguous().cuda()
    return q, k, v, q_r, kb, vb, Sb


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ra.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", [
    # (B, S, H, D, P, rank, causal, nsplit): a DiT-like share first, then a
    # smaller one with another head dimension, run count and causal mask
    [(1, 4096, 24, 128, 4, 0, False, 0), (1, 1024, 4, 64, 2, 1, True, 3)],
])
def test_noalloc_matches_workspace_split(case):
    for n, (B, S, H, D, P, rank, causal, nsplit) in enumerate(case):
        print(f"[gpu-test] noalloc call {n}: B={B} S={S} H={H} D={D} P={P} rank={rank} "
              f"causal={causal} nsplit={nsplit}", flush=True)
        q, k, v, q_r, kb, vb, Sb = _share(B, S, H, D, P, rank, causal, seed=11 + n)
        runs, ws_floats = ra.ring_split_plan(B, Sb, H, D, P, rank, causal, -1, nsplit)
        assert runs > 1, "the case must exercise the split"
        o_ref = torch.empty_like(q_r)
        l_ref = torch.empty((B, Sb, H), dtype=torch.float32, device="cuda")
        ra.ring_attn_fwd(q_r, kb, vb, rank, causal=causal, out=o_ref, lse_out=l_ref,
                         split=runs)
        o = torch.full_like(q_r, float("nan"))
        l = torch.full((B, Sb, H), float("nan"), dtype=torch.float32, device="cuda")
        ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o, l, causal=causal, nsplit=nsplit)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
        # and the bf16 bar against the oracle on sampled rows of every head
        rows = np.unique(np.linspace(0, Sb - 1, 48).astype(np.int64))
        klim = (rank + 1) * Sb if causal else S
        ref, _, _, _ = oracle.attention(q[:, rank * Sb:(rank + 1) * Sb], k[:, :klim], v[:, :klim],
                                        causal=causal, q_pos0=rank * Sb, rows=rows)
        c = oracle.compare(o[:, rows].cpu(), ref)
        print("[gpu-test]", {kk: f"{vv:.3e}" for kk, vv in c.items()}, flush=True)
        assert c["max_abs_err"] <= 1e-2 and c["cos"] > 0.999, c


def test_noalloc_refuses_plans_beyond_the_scratch():
    B, S, H, D, P, rank = 1, 4096, 24, 128, 4, 0
    q, k, v, q_r, kb, vb, Sb = _share(B, S, H, D, P, rank, False, seed=3)
    o = torch.empty_like(q_r)
    # 40 runs per query tile: 192 * 40 * 128 * 129 floats > 8 Mi
    runs, ws_floats = ra.ring_split_plan(B, Sb, H, D, P, rank, False, -1, 40)
    assert ws_floats > 8 * 2 ** 20
    with pytest.raises(RuntimeError, match="fixed scratch"):
        ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o, nsplit=40)
    with pytest.raises(RuntimeError, match="nsplit"):
        ra.ring_attn_fwd_split_noalloc(q_r, kb, vb, rank, o, nsplit=-1)
