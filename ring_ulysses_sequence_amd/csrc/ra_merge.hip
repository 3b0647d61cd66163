// Pairwise log-sum-exp merge of two partial attention results (the combine
// of [SPD] §四, the composable form of one ring round):
//   lse' = logaddexp(lse_acc, lse_blk)
//   o'   = o_acc * exp(lse_acc - lse') + o_blk * exp(lse_blk - lse')
// HBM-bound elementwise work: each row reads two D-vectors and two scalars
// and writes one D-vector and one scalar (plus the optional final copy).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "ra_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;

// One row is handled by D/4 consecutive lanes of ONE wavefront (D/4 divides
// 64), so every lane of a row reads lse_acc before any lane writes it.
__global__ __launch_bounds__(kThreads) void lse_merge(
    float* __restrict__ o_acc, float* lse_acc, const float* __restrict__ o_blk,
    const float* __restrict__ lse_blk, long long rows, int q4, void* o_final,
    int final_bf16) {
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / q4;
  if (row >= rows) return;
  const int c = (int)(t - row * q4);
  const float a = lse_acc[row];
  const float b = lse_blk[row];
  const float mx = fmaxf(a, b);
  float wa = 0.0f, wb = 0.0f, lse = -INFINITY;
  if (mx != -INFINITY) {
    // logaddexp via the larger term: lse = mx + ln(2^((a-mx)log2e) + 2^((b-mx)log2e))
    const float ea = __builtin_amdgcn_exp2f((a - mx) * kLog2e);
    const float eb = __builtin_amdgcn_exp2f((b - mx) * kLog2e);
    const float sum = ea + eb;
    lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
    const float inv = 1.0f / sum;
    wa = ea * inv;
    wb = eb * inv;
  }
  const float4 x = ((const float4*)o_acc)[t];
  const float4 y = ((const float4*)o_blk)[t];
  const float4 z = float4{fmaf(x.x, wa, y.x * wb), fmaf(x.y, wa, y.y * wb),
                          fmaf(x.z, wa, y.z * wb), fmaf(x.w, wa, y.w * wb)};
  ((float4*)o_acc)[t] = z;
  if (c == 0) lse_acc[row] = lse;
  if (o_final) {
    if (final_bf16) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 r;
      r[0] = (__bf16)z.x; r[1] = (__bf16)z.y; r[2] = (__bf16)z.z; r[3] = (__bf16)z.w;
      ((bf16x4*)o_final)[t] = r;
    } else {
      ((float4*)o_final)[t] = z;
    }
  }
}

// n-way form for a ring whose visited blocks were split over grid slices:
// slice s left its normalised partial in o_part[s] [rows, D] and its natural
// log-sum-exp in lse_part[s] [rows]; with L = log sum_s exp(lse_s),
//   o = sum_s exp(lse_s - L) o_s,   lse = L
// (slices that saw no key carry lse_s = -inf and weigh 0; a row no slice saw
// ends as (0, -inf)).  One row per D/4 consecutive lanes, as above.  NS is
// the slice count (all loads issued before any use), 0 for a run-time count.
template <int NS>
__global__ __launch_bounds__(kThreads) void split_merge(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int nsplit,
    long long rows, int q4, void* o, int out_bf16, float* lse_out) {
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / q4;
  if (row >= rows) return;
  const int c = (int)(t - row * q4);
  const int ns = NS > 0 ? NS : nsplit;
  constexpr int CAP = NS > 0 ? NS : 1;
  float ls[CAP];
  float4 xs[CAP];
  if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      ls[s] = lse_part[s * rows + row];
      xs[s] = ((const float4*)o_part)[s * rows * q4 + t];
    }
  }
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, NS > 0 ? ls[s] : lse_part[s * rows + row]);
  float4 acc = float4{0.0f, 0.0f, 0.0f, 0.0f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < ns; ++s) {
      const float l = NS > 0 ? ls[s] : lse_part[s * rows + row];
      const float4 x = NS > 0 ? xs[s] : ((const float4*)o_part)[s * rows * q4 + t];
      const float w = __builtin_amdgcn_exp2f((l - mx) * kLog2e);
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
      sum += w;
    }
    const float inv = 1.0f / sum;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
    lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
  }
  if (out_bf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 r;
    r[0] = (__bf16)acc.x; r[1] = (__bf16)acc.y; r[2] = (__bf16)acc.z; r[3] = (__bf16)acc.w;
    ((bf16x4*)o)[t] = r;
  } else {
    ((float4*)o)[t] = acc;
  }
  if (lse_out && c == 0) lse_out[row] = lse;
}

}  // namespace

extern "C" ra_status ra_ring_merge(float* o_acc, float* lse_acc, const float* o_blk,
                                   const float* lse_blk, int B, int Sq, int H, int D,
                                   void* o_final_opt, ra_dtype final_dt, void* stream) {
  static const char* name = "ra_ring_merge";
  ra::clear_error();
  if (B < 0 || Sq < 0 || H < 0 || D <= 0)
    return ra::fail(RA_ERR_SHAPE, "%s: need B, Sq, H >= 0 and D > 0", name);
  if (D % 4 != 0 || 64 % (D / 4) != 0)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: D=%d must be 4*2^k with D <= 256", name, D);
  if (final_dt != RA_BF16 && final_dt != RA_FP32)
    return ra::fail(RA_ERR_DTYPE, "%s: unknown final dtype %d", name, (int)final_dt);
  const long long rows = (long long)B * Sq * H;
  if (rows == 0) return RA_OK;
  if (!o_acc || !lse_acc || !o_blk || !lse_blk)
    return ra::fail(RA_ERR_NULL, "%s: NULL o/lse pointer", name);
  if (((uintptr_t)o_acc | (uintptr_t)o_blk | (uintptr_t)o_final_opt) & 15)
    return ra::fail(RA_ERR_SHAPE, "%s: o buffers must be 16-byte aligned", name);
  const int q4 = D / 4;
  const long long n = rows * q4;
  const long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return ra::fail(RA_ERR_UNSUPPORTED, "%s: too large", name);
  hipLaunchKernelGGL(lse_merge, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, o_acc, lse_acc, o_blk, lse_blk, rows, q4,
                     o_final_opt, final_dt == RA_BF16 ? 1 : 0);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}

namespace ra {

ra_status merge_splits(const char* name, const float* o_part, const float* lse_part, int nsplit,
                       long long rows, int D, void* o, ra_dtype dt, float* lse_opt,
                       void* stream) {
  const int q4 = D / 4;
  const long long n = rows * q4;
  const long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return ra::fail(RA_ERR_UNSUPPORTED, "%s: too large", name);
  if (blocks == 0) return RA_OK;
  const dim3 g((unsigned)blocks), t(kThreads);
  hipStream_t s = (hipStream_t)stream;
  const int bf = dt == RA_BF16 ? 1 : 0;
  switch (nsplit) {
    case 2: hipLaunchKernelGGL(split_merge<2>, g, t, 0, s, o_part, lse_part, 2, rows, q4, o, bf, lse_opt); break;
    case 3: hipLaunchKernelGGL(split_merge<3>, g, t, 0, s, o_part, lse_part, 3, rows, q4, o, bf, lse_opt); break;
    case 4: hipLaunchKernelGGL(split_merge<4>, g, t, 0, s, o_part, lse_part, 4, rows, q4, o, bf, lse_opt); break;
    default:
      hipLaunchKernelGGL(split_merge<0>, g, t, 0, s, o_part, lse_part, nsplit, rows, q4, o, bf,
                         lse_opt);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: merge launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}

}  // namespace ra
