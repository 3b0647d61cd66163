#!/usr/bin/env python3
"""Benchmark: attention TFLOP/s of one rank's ring-attention share on one GPU.

A step is one pass of the hot path over the long-context causal workload:
rank 3 of a P=8 ring over a global sequence of L=131072 tokens, 64 heads of
D=128 (hidden 8192), bf16 inputs with fp32 accumulation.  The rank's query
shard (16384 tokens) visits the 8 K/V blocks in ring order 3,2,1,0,7,6,5,4:
its own block is diagonal (element mask), blocks 2,1,0 are fully visible,
blocks 7..4 are in the future and never read.  One step = one launch of the
fused ring kernel (ra_ring_attn_fwd), inputs resident in HBM.

Algorithmic work = 4*D FLOPs per visible (query, key) pair (2D for Q K^T,
2D for P V), summed over heads and the share's rows; masked pairs, skipped
blocks and softmax exponentials are not counted.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints ONE JSON line.  One GPU only: --gpus N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention TFLOP/s per GPU (bf16, per-rank shard) + % of MFMA peak"


def visible_pairs_causal_rank(rank: int, Sb: int, valid_len: int) -> int:
    """Number of visible (query, key) pairs of a causal rank share per head:
    query at global position p (< valid_len) sees keys 0..p."""
    lo = rank * Sb
    hi = min((rank + 1) * Sb, valid_len)
    if hi <= lo:
        return 0
    # sum_{p=lo}^{hi-1} (p + 1)
    return (lo + 1 + hi) * (hi - lo) // 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the side measurements (Ulysses layout, DiT shard)")
    ap.add_argument("--attn-kernel", choices=["auto", "rowmax"], default="auto",
                    help="how the bf16 kernel keeps the row max (both compute the same result)")
    return ap.parse_args()


KERNEL_NAMES = {"auto": "ring_attn_bf16<128,8,false>", "rowmax": "ring_attn_bf16<128,8,false>"}
ATTN_SOURCE = os.path.join(ROOT, "ring_ulysses_sequence_amd", "csrc", "ra_attn.hip")


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` on this workload, from the committed
    rocprofv3 counter summary under profiles/ -- only if the summary was taken
    on the attention source as it is now (its sha256 matches); else None."""
    import glob
    import hashlib
    sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        for line in open(path, encoding="utf-8"):
            if not line.startswith("traffic_per_launch:"):
                continue
            kv = dict(item.split("=", 1) for item in line.split(":", 1)[1].split())
            if kv.get("kernel") == kernel and kv.get("source_sha256") == sha:
                return int(kv["bytes"]), os.path.relpath(path, ROOT)
    return None, None


def cpu_baseline(q, k, v, rank, Sb, H, D, n_rows=512):
    """The fp64 oracle, as it stands, on a bounded sample of the same share:
    n_rows evenly spaced query rows of rank 3, all 64 heads, each over its
    whole visible prefix (about 15 s of host time).  Returns the oracle's
    algorithmic TFLOP/s on it."""
    import numpy as np
    import oracle
    rows = np.unique(np.linspace(0, Sb - 1, n_rows).astype(np.int64))
    kq = k[:, :(rank + 1) * Sb].cpu()
    vq = v[:, :(rank + 1) * Sb].cpu()
    qr = q[:, rank * Sb:(rank + 1) * Sb].cpu()
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads") or 0) for i in libs) or None
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs) or None
    except Exception:
        pass
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    t0 = time.perf_counter()
    oracle.attention(qr, kq, vq, causal=True, q_pos0=rank * Sb, k_pos0=0, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int(sum(rank * Sb + int(r) + 1 for r in rows)) * H
    flops = 4.0 * D * pairs
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
        "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
        "host_logical_cpus": os.cpu_count(),
        "sample": f"rank {rank} share, {len(rows)} evenly spaced query rows x {H} heads, "
                  f"each over its full causal prefix ({flops:.3e} algorithmic FLOPs, "
                  f"{dt:.1f} s, numpy fp64)",
        "seconds": dt,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the ring on ONE GPU; the library has "
              "no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import ring_ulysses_sequence_amd as ra
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ra.lib()
    ra.set_attn_kernel({"auto": ra.RA_KERNEL_AUTO, "rowmax": ra.RA_KERNEL_ROWMAX}[args.attn_kernel])
    w = W.LONG_CAUSAL
    rank, Sb, H, D, P = 3, w.block_len, w.H, w.D, w.P
    q, k, v = W.make_qkv(w, device="cuda")
    kb = [k[:, j * Sb:(j + 1) * Sb] for j in range(P)]   # B = 1: contiguous blocks
    vb = [v[:, j * Sb:(j + 1) * Sb] for j in range(P)]
    q_r = q[:, rank * Sb:(rank + 1) * Sb]
    o = torch.empty_like(q_r)
    lse = torch.empty((1, Sb, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        ra.ring_attn_fwd(q_r, kb, vb, rank, causal=True, valid_len=w.S, out=o,
                         lse_out=lse, stream=stream)

    pairs = visible_pairs_causal_rank(rank, Sb, w.S) * H * w.B
    flops = 4.0 * D * pairs

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-launch HIP events on the launch stream (the roofline's duration)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12

    kernel = KERNEL_NAMES[args.attn_kernel]
    traffic, traffic_src = measured_traffic(kernel)
    # Q, the four visited K and V blocks, O (bf16) and lse (fp32)
    algo_bytes = (q_r.numel() * 2 + 4 * 2 * kb[0].numel() * 2 + o.numel() * 2
                  + lse.numel() * 4)
    extra = {}
    if not args.no_extra:
        extra = side_measurements(torch, ra, W, stream)
        extra.update(config_measurements(torch, ra, W, stream))
        extra.update(zigzag_measurements(torch, ra, W, stream, q, k, v))
        extra.update(backward_measurement(torch, ra, W, stream, q_r, kb, vb, o, lse, flops))
        extra.update(gqa_varlen_measurements(torch, ra, stream, q_r, k, v, kb, vb))
        extra.update(composable_measurements(torch, ra, stream, q_r, kb, vb, flops))
        extra.update(gemm_reference(torch, stream))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, rank, Sb, H, D)
        extra["cpu_baseline_seconds"] = round(cpu.pop("seconds"), 2)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) q,k,v (seed 0, torch device generator) cast to bf16",
        "config": {
            "workload": "long-context causal ring share: L=131072, H=64, D=128 "
                        "(hidden 8192), P=8, rank 3 (16384 query tokens over K/V "
                        "blocks 3,2,1,0; 7..4 skipped), B=1",
            "global_batch": 1, "seq_len": w.S, "heads": H, "head_dim": D, "ring_degree": P,
            "rank": rank, "causal": True, "parallelism": "one rank's share on 1 GPU",
            "attn_kernel": args.attn_kernel,
            "algorithmic_flops_per_step": flops,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma", "kernel": kernel,
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(avg_launch_ms, 4),
            "median_launch_ms": round(sorted(launch_ms)[len(launch_ms) // 2], 4),
            "min_launch_ms": round(min(launch_ms), 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM/fabric, rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-kernel calibrated)",
            "traffic_source": traffic_src,
            "algorithmic_bytes": algo_bytes,
        },
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 3),
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


def config_measurements(torch, ra, W, stream):
    """Side numbers for the other configurations, not the step: the Ulysses
    local attention (all eight ranks' head shards in one launch) and the
    whole Ulysses path (three seq->head transposes, attention, head->seq);
    every rank of the padded causal share in sequence; the tiny fp32 ring
    (launch-latency bound)."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(f, n):
        for _ in range(3):
            f()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # Ulysses: [8, 1, 2048, 32, 128] per tensor; attention on 4 heads per rank
    w = W.ULYSSES
    P, Sl, Hl = w.P, w.S // w.P, w.H // w.P
    q, k, v = W.make_qkv(w, device="cuda")
    stack = lambda x: x.view(w.B, P, Sl, w.H, w.D).transpose(0, 1).contiguous()
    qs, ks, vs = stack(q), stack(k), stack(v)
    del q, k, v
    qh, kh, vh = ra.seq2head(qs), ra.seq2head(ks), ra.seq2head(vs)
    flat = lambda x: x.view(P * w.B, w.S, Hl, w.D)
    oh = torch.empty_like(flat(qh))
    attn = lambda: ra.ring_attn_fwd(flat(qh), [flat(kh)], [flat(vh)], 0, out=oh,
                                    want_lse=False, stream=stream)
    ms = timed(attn, 10)
    fl = 4.0 * w.D * w.S * w.S * w.H * w.B
    out["ulysses_attention_all_ranks"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
                                          "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    osq = torch.empty_like(qs)

    def path():
        ra.seq2head(qs, out=qh, stream=stream)
        ra.seq2head(ks, out=kh, stream=stream)
        ra.seq2head(vs, out=vh, stream=stream)
        attn()
        ra.head2seq(oh.view(P, w.B, w.S, Hl, w.D), out=osq, stream=stream)
    ms = timed(path, 10)
    out["ulysses_path_all_ranks"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2)}
    del qs, ks, vs, qh, kh, vh, oh, osq

    # padded causal share (S = 3000 in 3008, P = 4): every rank in turn
    w = W.PADDED_CAUSAL
    Sb = w.block_len
    q, k, v = W.make_qkv(w, device="cuda")
    kb = [k[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    vb = [v[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    qr = [q[:, r * Sb:(r + 1) * Sb].contiguous() for r in range(w.P)]
    outs = [torch.empty_like(x) for x in qr]
    ranks = lambda: [ra.ring_attn_fwd(qr[r], kb, vb, r, causal=True, valid_len=w.S, out=outs[r],
                                      want_lse=False, stream=stream) for r in range(w.P)]
    ms = timed(ranks, 20)
    # visible (query, key) pairs over the real rows: sum of (i + 1) for i < S
    fl = 4.0 * w.D * w.H * w.B * w.S * (w.S + 1) / 2
    out["padded_causal_all_ranks"] = {"ms": round(ms, 4), "us_per_rank": round(1e3 * ms / w.P, 2),
                                      "tflops": round(fl / ms / 1e9, 2)}
    # the same four calls replayed from a HIP graph: the GPU's own time,
    # without the Python binding's per-call host work between launches
    ref = [x.clone() for x in outs]
    gms = graph_ms(torch, lambda: [ra.ring_attn_fwd(qr[r], kb, vb, r, causal=True, valid_len=w.S,
                                                    out=outs[r], want_lse=False)
                                   for r in range(w.P)], outs, ref, 20)
    if gms is not None:
        out["padded_causal_all_ranks"].update({"graph_ms": round(gms, 4),
                                               "graph_us_per_rank": round(1e3 * gms / w.P, 2),
                                               "graph_tflops": round(fl / gms / 1e9, 2)})
    del q, k, v, kb, vb, qr, outs

    # tiny fp32 ring (B = 1, S = 256, H = 2, D = 64, P = 2): both ranks
    w = W.TINY_FP32
    Sb = w.block_len
    q, k, v = W.make_qkv(w, device="cuda")
    kb = [k[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    vb = [v[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    qr = [q[:, r * Sb:(r + 1) * Sb].contiguous() for r in range(w.P)]
    outs = [torch.empty_like(x) for x in qr]
    ms = timed(lambda: [ra.ring_attn_fwd(qr[r], kb, vb, r, out=outs[r], want_lse=False,
                                         stream=stream) for r in range(w.P)], 50)
    out["tiny_fp32_both_ranks"] = {"ms": round(ms, 4), "us_per_rank": round(1e3 * ms / w.P, 2)}
    ref = [x.clone() for x in outs]
    gms = graph_ms(torch, lambda: [ra.ring_attn_fwd(qr[r], kb, vb, r, out=outs[r], want_lse=False)
                                   for r in range(w.P)], outs, ref, 50)
    if gms is not None:
        out["tiny_fp32_both_ranks"].update({"graph_ms": round(gms, 4),
                                            "graph_us_per_rank": round(1e3 * gms / w.P, 2)})
    return out


def graph_ms(torch, calls, outs, ref, n):
    """Average time of `calls` replayed from a captured HIP graph (None if it
    cannot be captured); every replay's outputs must equal the eager ones."""
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            calls()  # warm the graph pool's allocations outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            calls()
    except Exception as e:  # capture is a convenience for timing only
        print(f"graph capture failed: {e}", file=sys.stderr, flush=True)
        return None
    for _ in range(3):
        for x in outs:
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, ref):
            if not torch.equal(x, y):
                raise RuntimeError("graph replay differs from the eager result")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def gemm_reference(torch, stream, n=8192, reps=30):
    """A reference point for the board's dense bf16 matrix-core throughput
    at its power limit, outside this library: torch.matmul (hipBLASLt) on
    random N(0,1) bf16 operands of n x n x n, timed over `reps` products
    after a warmup long enough for the clock to settle.  Context for the
    attention figure, not part of the step."""
    g = torch.Generator(device="cuda").manual_seed(1)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        for _ in range(10):
            torch.matmul(a, b, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / ms / 1e9
    return {"gemm_bf16_reference": {"n": n, "ms": round(ms, 4), "tflops": round(tf, 1),
                                    "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                                    "library": "torch.matmul (hipBLASLt), N(0,1) operands"}}


def side_measurements(torch, ra, W, stream):
    """Side numbers, not the step: the DiT-shard ring (rank 0; split as the
    library plans, which the binding does by default) and the
    Ulysses seq->head / head->seq layout of one tensor."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # DiT shard, rank 0 (non-causal, 4 blocks of 1024)
    w = W.DIT_SHARD
    q, k, v = W.make_qkv(w, device="cuda")
    Sb = w.block_len
    kb = [k[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    vb = [v[:, j * Sb:(j + 1) * Sb].contiguous() for j in range(w.P)]
    q0 = q[:, :Sb].contiguous()
    o = torch.empty_like(q0)
    for _ in range(3):
        ra.ring_attn_fwd(q0, kb, vb, 0, out=o, want_lse=False, stream=stream)
    a, b = ev(), ev()
    n = 50
    a.record(stream)
    for _ in range(n):
        ra.ring_attn_fwd(q0, kb, vb, 0, out=o, want_lse=False, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    fl = 4.0 * w.D * Sb * w.S * w.H * w.B
    out["dit_shard_rank0"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
                              "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                              "split_runs_per_query_tile":
                                  ra.ring_split_plan(w.B, Sb, w.H, w.D, w.P, 0)[0]}
    del q, k, v, kb, vb, q0, o
    # Ulysses layout: [8, 1, 2048, 32, 128] bf16 tensors each way.  Three
    # tensors are used in turn (384 MiB, more than the 256 MB last-level
    # cache), so every call reads a source that is not cached: the HBM-bound
    # figure.  "warm_*" repeats one tensor, whose source then stays cached.
    w = W.ULYSSES
    xs = [W.random_tensor((w.P, w.B, w.S // w.P, w.H, w.D), seed=s, device="cuda")
          for s in range(3)]
    ys = [ra.seq2head(x, stream=stream) for x in xs]
    zs = [ra.head2seq(y, stream=stream) for y in ys]
    torch.cuda.synchronize()
    for name, fn, srcs, dsts in (("seq2head", ra.seq2head, xs, ys),
                                 ("head2seq", ra.head2seq, ys, zs)):
        byts = 2.0 * srcs[0].numel() * srcs[0].element_size()
        rec = {}
        for tag, k in (("", 3), ("warm_", 1)):
            a, b = ev(), ev()
            a.record(stream)
            for i in range(n):
                fn(srcs[i % k], out=dsts[i % k], stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / n
            rec.update({f"{tag}ms": round(ms, 4), f"{tag}GBps": round(byts / ms / 1e6, 1),
                        f"{tag}frac_hbm": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)})
        out[f"ulysses_{name}"] = rec
    # the practical copy ceiling of the board for comparison: a library
    # device-to-device copy (torch copy_) of the same tensors, same rotation
    a, b = ev(), ev()
    with torch.cuda.stream(stream):
        for i in range(3):
            ys[i].view(-1).copy_(xs[i].view(-1))
        a.record(stream)
        for i in range(n):
            ys[i % 3].view(-1).copy_(xs[i % 3].view(-1))
        b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    byts = 2.0 * xs[0].numel() * xs[0].element_size()
    out["copy_reference"] = {"ms": round(ms, 4), "GBps": round(byts / ms / 1e6, 1),
                             "frac_hbm": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3),
                             "library": "torch copy_ (device to device), same three tensors"}
    del xs, ys, zs
    return out


def backward_measurement(torch, ra, W, stream, q_r, kb, vb, o, lse, fwd_flops):
    """The ring backward of the same rank-3 share (dq and the dk/dv parts of
    the four visited blocks, accumulated into preallocated fp32 buffers).
    Algorithmic FLOPs: 2.5x the forward's (five products of 2*D per visible
    pair: the recomputed scores, dP, dV, dK, dQ)."""
    do = W.random_tensor(q_r.shape, seed=41, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    dq = torch.zeros(q_r.shape, **f32)
    # blocks 4..7 are skipped (causal future) and their buffers never
    # touched, so block 0's buffers stand in for them
    dk = [torch.zeros(q_r.shape, **f32) for _ in range(4)]
    dv = [torch.zeros(q_r.shape, **f32) for _ in range(4)]
    dk += [dk[0]] * (len(kb) - 4)
    dv += [dv[0]] * (len(kb) - 4)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def run():
        ra.ring_attn_bwd(q_r, kb, vb, o, do, lse, 3, causal=True, dq=dq, dk_blocks=dk,
                         dv_blocks=dv, stream=stream)
    run()
    torch.cuda.synchronize()
    n = 3
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(n):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    fl = 2.5 * fwd_flops
    return {"backward_long_rank3": {"ms": round(ms, 3), "flops": fl,
                                    "tflops": round(fl / ms / 1e9, 2),
                                    "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}}


def packed_sample_bounds(S: int, n: int, seed: int):
    """Boundaries of n packed samples covering [0, S): lengths drawn from a
    seeded uniform split (the synthetic stand-in for a mixed-length batch)."""
    import numpy as np
    g = np.random.default_rng(seed)
    cuts = np.sort(g.choice(np.arange(1, S), size=n - 1, replace=False))
    return [0] + [int(x) for x in cuts] + [S]


def composable_measurements(torch, ra, stream, q_r, kb, vb, fwd_flops):
    """The composable form of the same rank-3 share (one launch per visited
    block in ring order: block_attn_fwd for the first, block_attn_fwd_acc
    folding each later one into the running partial in its own epilogue,
    the last one writing bf16; four rounds, no separate merge launch), its
    ratio to the fused ring measured beside it, and one ring_merge on the
    share's fp32 partials alone, in GB/s of its algorithmic bytes: per
    (b, s, h) row it reads two fp32 O rows and two lse and writes one O row
    and one lse, 2*D*4 + 8 + D*4 + 4 bytes."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    B, Sb, H, D = q_r.shape
    rank = 3

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {}
    ms = timed(lambda: ra.ring_attn_composable(q_r, kb, vb, rank, causal=True, stream=stream), 3)
    ms_f = timed(lambda: ra.ring_attn_fwd(q_r, kb, vb, rank, causal=True, stream=stream), 3)
    out["composable_long_rank3"] = {"ms": round(ms, 3), "tflops": round(fwd_flops / ms / 1e9, 2),
                                    "rounds": 4, "fused_ms": round(ms_f, 3),
                                    "vs_fused": round(ms / ms_f, 4)}
    o_acc, lse_acc, _, _ = ra.block_attn_fwd(q_r, kb[2], vb[2], q_pos0=rank * Sb, k_pos0=2 * Sb,
                                             causal=True, want_ml=False, stream=stream)
    o_blk, lse_blk, _, _ = ra.block_attn_fwd(q_r, kb[1], vb[1], q_pos0=rank * Sb, k_pos0=1 * Sb,
                                             causal=True, want_ml=False, stream=stream)
    ms = timed(lambda: ra.ring_merge(o_acc, lse_acc, o_blk, lse_blk, stream=stream), 20)
    rows = B * Sb * H
    byts = rows * (2 * D * 4 + 8 + D * 4 + 4)
    out["ring_merge_long_rank3"] = {"ms": round(ms, 4), "bytes": byts,
                                    "GBps": round(byts / ms / 1e6, 1),
                                    "frac_hbm": round(byts / ms / 1e6 / PEAK_HBM_GBS, 3)}
    del o_acc, lse_acc, o_blk, lse_blk
    return out


def gqa_varlen_measurements(torch, ra, stream, q_r, k, v, kb, vb):
    """The same rank-3 share with grouped-query K/V (8 K/V heads for the 64
    query heads: the first head of each group of 8) and as a packed sequence
    of 16 samples (causal within each sample), each with its own algorithmic
    FLOPs (4*D per visible pair)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    B, Sb, H, D = q_r.shape
    P, rank = len(kb), 3

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {}
    Hkv = 8
    kg = k[:, :, ::H // Hkv].contiguous()
    vg = v[:, :, ::H // Hkv].contiguous()
    kgb = [kg[:, j * Sb:(j + 1) * Sb] for j in range(P)]
    vgb = [vg[:, j * Sb:(j + 1) * Sb] for j in range(P)]
    o = torch.empty_like(q_r)
    ms = timed(lambda: ra.ring_attn_fwd(q_r, kgb, vgb, rank, causal=True, out=o, want_lse=False,
                                        stream=stream))
    fl = 4.0 * D * H * visible_pairs_causal_rank(rank, Sb, P * Sb)
    out["gqa_long_rank3_hkv8"] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 2),
                                  "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    del kg, vg, kgb, vgb
    cu = packed_sample_bounds(P * Sb, 16, seed=5)
    q0, q1 = rank * Sb, (rank + 1) * Sb
    pairs = 0
    for s0, s1 in zip(cu[:-1], cu[1:]):
        a, b = max(s0, q0), min(s1, q1)
        if b > a:  # query p sees keys s0 .. p of its sample
            pairs += (a - s0 + 1 + b - s0) * (b - a) // 2
    fl = 4.0 * D * H * pairs
    ms = timed(lambda: ra.ring_attn_fwd_varlen(q_r, kb, vb, rank, cu, causal=True, out=o,
                                               want_lse=False, stream=stream))
    out["varlen_long_rank3_16_samples"] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 2),
                                           "flops": fl, "samples": cu}
    return out


def zigzag_measurements(torch, ra, W, stream, q, k, v):
    """Load balance of the causal ring on the same long-context tensors: the
    zigzag shares of ranks 0 and 7 (chunks r and 15-r of 8192 rows, equal
    work) against the slowest contiguous rank (7, 7.5 blocks of work).  The
    ring job takes as long as its slowest rank."""
    w = W.LONG_ZIGZAG
    P, c, H, D = w.P, w.S // (2 * w.P), w.H, w.D
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def share(x, r):
        a, b = r, 2 * P - 1 - r
        return torch.cat([x[:, a * c:(a + 1) * c], x[:, b * c:(b + 1) * c]], dim=1).contiguous()

    ks = [share(k, r) for r in range(P)]
    vs = [share(v, r) for r in range(P)]

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {}
    zz_flops = 4.0 * D * H * c * (2 * P * c + 1)
    for r in w.ranks:
        q_r = share(q, r)
        o = torch.empty_like(q_r)
        ms = timed(lambda: ra.zigzag_attn_fwd(q_r, ks, vs, r, causal=True, out=o,
                                              want_lse=False, stream=stream))
        out[f"zigzag_long_rank{r}"] = {"ms": round(ms, 3), "flops": zz_flops,
                                       "tflops": round(zz_flops / ms / 1e9, 2)}
        if r == w.ranks[-1]:
            # the zigzag backward of the same share (five products per pair)
            o, lse = ra.zigzag_attn_fwd(q_r, ks, vs, r, causal=True, stream=stream)
            do = torch.randn(q_r.shape, generator=torch.Generator(device="cuda").manual_seed(43),
                             device="cuda").to(q_r.dtype)
            f32 = dict(dtype=torch.float32, device="cuda")
            dq = torch.zeros(q_r.shape, **f32)
            dks = [torch.zeros(q_r.shape, **f32) for _ in range(P)]
            dvs = [torch.zeros(q_r.shape, **f32) for _ in range(P)]
            ms = timed(lambda: ra.zigzag_attn_bwd(q_r, ks, vs, o, do, lse, r, causal=True, dq=dq,
                                                  dk_shares=dks, dv_shares=dvs, stream=stream))
            out[f"zigzag_backward_long_rank{r}"] = {
                "ms": round(ms, 3), "flops": 2.5 * zz_flops,
                "tflops": round(2.5 * zz_flops / ms / 1e9, 2)}
            del lse, do, dq, dks, dvs
        del q_r, o
    del ks, vs
    Sb = w.S // P
    kb = [k[:, j * Sb:(j + 1) * Sb] for j in range(P)]
    vb = [v[:, j * Sb:(j + 1) * Sb] for j in range(P)]
    q7 = q[:, 7 * Sb:8 * Sb]
    o = torch.empty_like(q7)
    ms = timed(lambda: ra.ring_attn_fwd(q7, kb, vb, 7, causal=True, out=o, want_lse=False,
                                        stream=stream))
    fl7 = 4.0 * D * H * visible_pairs_causal_rank(7, Sb, w.S)
    out["contiguous_long_rank7"] = {"ms": round(ms, 3), "flops": fl7,
                                    "tflops": round(fl7 / ms / 1e9, 2)}
    slow_zz = max(out[f"zigzag_long_rank{r}"]["ms"] for r in w.ranks)
    out["zigzag_job_speedup_vs_contiguous"] = round(ms / slow_zz, 3)
    return out


if __name__ == "__main__":
    main()
