// Ulysses sequence-shard <-> head-shard transposes ([RA] §3.5) on one GPU.
//
// The P per-rank tensors are stacked rank-major.  With Sl = S/P, Hl = H/P:
//   seq2head: dst[r, b, j*Sl + s, h', d] = src[j, b, s, r*Hl + h', d]
//   head2seq: dst[j, b, s, r*Hl + h', d] = src[r, b, j*Sl + s, h', d]
// For fixed (rank, batch, token) the Hl*D elements of one head group are
// contiguous on both sides, so both maps are copies of "runs" of
// Hl*D*elem_bytes bytes between computed offsets.  The kernels walk the
// destination in order (coalesced stores), read whole runs (coalesced
// loads), move raw bits only, and are HBM-bound: every byte is read once
// and written once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ra_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte units per thread

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// seq2head: destination run (r, b, t) with t in [0, S) -> source run
// (j = t / Sl, b, s = t % Sl, head group r); one run per destination row.
__device__ __forceinline__ long long s2h_src_run(long long dst_run, int P, int B,
                                                 long long S, long long Sl) {
  const long long t = dst_run % S;
  const long long rb = dst_run / S;
  const long long b = rb % B;
  const long long r = rb / B;
  const long long j = t / Sl, s = t % Sl;
  // source rows (j, b, s) hold P runs each; run r within the row
  return ((j * B + b) * Sl + s) * P + r;
}

// head2seq: destination run (j, b, s, r) -> source run (r, b, j*Sl + s).
__device__ __forceinline__ long long h2s_src_run(long long dst_run, int P, int B,
                                                 long long S, long long Sl) {
  const long long r = dst_run % P;
  const long long row = dst_run / P;  // (j, b, s)
  const long long s = row % Sl;
  const long long jb = row / Sl;
  const long long b = jb % B;
  const long long j = jb / B;
  return (r * B + b) * S + j * Sl + s;
}

// Vector path for any run of a whole number of 16-byte units (64-bit
// index arithmetic per unit).
template <bool kSeq2Head>
__global__ __launch_bounds__(kThreads) void permute_vec16(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, long long n_units,
    int units_per_run, int P, int B, long long S, long long Sl) {
  const long long base =
      ((long long)blockIdx.x * kThreads * kUnroll) + threadIdx.x;
  u32x4 buf[kUnroll];
  long long idx[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const long long du = base + (long long)u * kThreads;
    idx[u] = du;
    if (du < n_units) {
      const long long run = du / units_per_run;
      const int c = (int)(du - run * units_per_run);
      const long long sr = kSeq2Head ? s2h_src_run(run, P, B, S, Sl)
                                     : h2s_src_run(run, P, B, S, Sl);
      buf[u] = __builtin_nontemporal_load(&src[sr * units_per_run + c]);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (idx[u] < n_units) __builtin_nontemporal_store(buf[u], &dst[idx[u]]);
}

// 32-bit forms of the run maps, for tensors of fewer than 2^31 units.
__device__ __forceinline__ unsigned s2h_src_run32(unsigned dst_run, unsigned P, unsigned B,
                                                  unsigned S, unsigned Sl) {
  const unsigned t = dst_run % S, rb = dst_run / S;
  const unsigned b = rb % B, r = rb / B;
  const unsigned j = t / Sl, s = t % Sl;
  return ((j * B + b) * Sl + s) * P + r;
}
__device__ __forceinline__ unsigned h2s_src_run32(unsigned dst_run, unsigned P, unsigned B,
                                                  unsigned S, unsigned Sl) {
  const unsigned r = dst_run % P, row = dst_run / P;
  const unsigned s = row % Sl, jb = row / Sl;
  const unsigned b = jb % B, j = jb / B;
  return (r * B + b) * S + j * Sl + s;
}

// Vector path by 1 KiB pieces: each wave moves kPieces pieces of 64
// consecutive destination units (one unit per lane), all loads before the
// stores.  Runs are a multiple of 64 units (a piece lies in one run) or
// divide 64 (a piece covers 64 / units_per_run whole runs), so the index
// arithmetic is a handful of 32-bit divisions per piece, not per unit.
// Loads and stores are non-temporal: each byte is touched once.  Measured on
// 128 MiB tensors whose source is not cached (three tensors in turn, more
// than the 256 MB last-level cache): one piece per wave with non-temporal
// loads 44 us each way, against 46-52 us with ordinary loads or four pieces
// per wave.  (A source still in that cache reads faster with ordinary
// loads: 39 us.)
constexpr int kPieces = 1;
template <bool kSeq2Head>
__global__ __launch_bounds__(kThreads) void permute_pieces(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, unsigned n_units,
    unsigned units_per_run, unsigned P, unsigned B, unsigned S, unsigned Sl) {
  const unsigned lane = threadIdx.x & 63;
  const unsigned piece0 = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * kPieces;
  u32x4 buf[kPieces];
  unsigned di[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const unsigned du = (piece0 + u) * 64 + lane;
    di[u] = du;
    if (du < n_units) {
      const unsigned run = du / units_per_run;
      const unsigned c = du - run * units_per_run;
      const unsigned sr = kSeq2Head ? s2h_src_run32(run, P, B, S, Sl)
                                    : h2s_src_run32(run, P, B, S, Sl);
      buf[u] = __builtin_nontemporal_load(&src[(size_t)sr * units_per_run + c]);
    }
  }
#pragma unroll
  for (int u = 0; u < kPieces; ++u)
    if (di[u] < n_units) __builtin_nontemporal_store(buf[u], &dst[di[u]]);
}

// Element path: any run length, element of T (1, 2, 4 or 8 bytes).
template <bool kSeq2Head, typename T>
__global__ __launch_bounds__(kThreads) void permute_elem(
    const T* __restrict__ src, T* __restrict__ dst, long long n_elems,
    int elems_per_run, int P, int B, long long S, long long Sl) {
  const long long de = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (de >= n_elems) return;
  const long long run = de / elems_per_run;
  const int c = (int)(de - run * elems_per_run);
  const long long sr = kSeq2Head ? s2h_src_run(run, P, B, S, Sl)
                                 : h2s_src_run(run, P, B, S, Sl);
  dst[de] = src[sr * elems_per_run + c];
}

template <bool kSeq2Head, typename T>
hipError_t launch_elem(const void* src, void* dst, long long n_elems,
                       int elems_per_run, int P, int B, long long S,
                       long long Sl, hipStream_t stream) {
  const long long blocks = (n_elems + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((permute_elem<kSeq2Head, T>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, stream, (const T*)src, (T*)dst, n_elems,
                     elems_per_run, P, B, S, Sl);
  return hipGetLastError();
}

template <bool kSeq2Head>
ra_status permute(const char* name, const void* src, void* dst, int P, int B,
                  long long S, int H, int D, int elem_bytes, void* stream_) {
  ra::clear_error();
  if (P <= 0 || B < 0 || S < 0 || H <= 0 || D <= 0)
    return ra::fail(RA_ERR_SHAPE, "%s: need P, H, D > 0 and B, S >= 0", name);
  if (S % P != 0)
    return ra::fail(RA_ERR_SHAPE,
                    "%s: sequence length %lld is not divisible by P=%d; pad it "
                    "to %lld (ra_padded_len)", name, S, P,
                    (S + (long long)P * RA_PAD_MULTIPLE - 1) /
                        ((long long)P * RA_PAD_MULTIPLE) * P * RA_PAD_MULTIPLE);
  if (H % P != 0)
    return ra::fail(RA_ERR_SHAPE,
                    "%s: head count H=%d is not divisible by P=%d", name, H, P);
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return ra::fail(RA_ERR_DTYPE, "%s: elem_bytes must be 1, 2, 4 or 8 (got %d)",
                    name, elem_bytes);
  const long long Sl = S / P;
  const int Hl = H / P;
  const long long run_bytes = (long long)Hl * D * elem_bytes;
  if (run_bytes > (1LL << 30))
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: head-group run too long", name);
  const long long n_runs = (long long)P * B * S;
  if (n_runs == 0) return RA_OK;
  if (!src || !dst) return ra::fail(RA_ERR_NULL, "%s: NULL src or dst", name);
  // ranges of src and dst are both n_runs * run_bytes
  const long long total = n_runs * run_bytes;
  const char* s0 = (const char*)src;
  const char* d0 = (const char*)dst;
  if (s0 < d0 + total && d0 < s0 + total)
    return ra::fail(RA_ERR_SHAPE, "%s: src and dst overlap", name);
  hipStream_t stream = (hipStream_t)stream_;
  hipError_t err;
  const bool vec = run_bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 &&
                   ((uintptr_t)dst % 16) == 0;
  const long long upr16 = run_bytes / 16;
  if (vec && (upr16 % 64 == 0 || 64 % upr16 == 0) && n_runs * upr16 < (1LL << 31)) {
    const long long n_units = n_runs * upr16;
    const long long per_block = (long long)kThreads * kPieces;
    const long long blocks = (n_units + per_block - 1) / per_block;
    hipLaunchKernelGGL((permute_pieces<kSeq2Head>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, (const u32x4*)src, (u32x4*)dst, (unsigned)n_units,
                       (unsigned)upr16, (unsigned)P, (unsigned)B, (unsigned)S, (unsigned)Sl);
    err = hipGetLastError();
  } else if (vec) {
    const int units_per_run = (int)(run_bytes / 16);
    const long long n_units = n_runs * units_per_run;
    const long long per_block = (long long)kThreads * kUnroll;
    const long long blocks = (n_units + per_block - 1) / per_block;
    if (blocks > 0x7fffffffLL)
      return ra::fail(RA_ERR_UNSUPPORTED, "%s: tensor too large", name);
    hipLaunchKernelGGL((permute_vec16<kSeq2Head>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, (const u32x4*)src,
                       (u32x4*)dst, n_units, units_per_run, P, B, S, Sl);
    err = hipGetLastError();
  } else {
    const int epr = Hl * D;
    const long long n_elems = n_runs * epr;
    if ((n_elems + kThreads - 1) / kThreads > 0x7fffffffLL)
      return ra::fail(RA_ERR_UNSUPPORTED, "%s: tensor too large", name);
    switch (elem_bytes) {
      case 1: err = launch_elem<kSeq2Head, uint8_t>(src, dst, n_elems, epr, P, B, S, Sl, stream); break;
      case 2: err = launch_elem<kSeq2Head, uint16_t>(src, dst, n_elems, epr, P, B, S, Sl, stream); break;
      case 4: err = launch_elem<kSeq2Head, uint32_t>(src, dst, n_elems, epr, P, B, S, Sl, stream); break;
      default: err = launch_elem<kSeq2Head, uint64_t>(src, dst, n_elems, epr, P, B, S, Sl, stream); break;
    }
  }
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}

}  // namespace

extern "C" ra_status ra_seq2head(const void* src, void* dst, int P, int B,
                                 long long S, int H, int D, int elem_bytes,
                                 void* stream) {
  return permute<true>("ra_seq2head", src, dst, P, B, S, H, D, elem_bytes, stream);
}

extern "C" ra_status ra_head2seq(const void* src, void* dst, int P, int B,
                                 long long S, int H, int D, int elem_bytes,
                                 void* stream) {
  return permute<false>("ra_head2seq", src, dst, P, B, S, H, D, elem_bytes, stream);
}
