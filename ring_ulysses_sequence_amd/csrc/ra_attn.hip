// Ring-order block attention on CDNA4 (gfx950): the local query shard stays
// on chip while K/V blocks stream through LDS in ring order, merged by the
// online-softmax recurrence ([RA] §3.2-§3.4).
//
// One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
// wave owns 32 rows.  Per K/V tile of 64 keys a wave computes the TRANSPOSED
// score tile S^T = K Q^T on the matrix cores, so that every lane holds the
// scores of one query column: the row max and row sum are in-lane reductions
// plus one cross-half exchange (v_permlane32_swap), not 32-lane butterflies.
// The probabilities P^T then feed O^T += V^T P^T directly as the B operand,
// which needs V^T in LDS; V is transposed while it is staged.
//
// Matrix-core operand layouts used below (64-lane wave, l = lane,
// col = l % 32, half = l / 32):
//   32x32x16 bf16  A[m][k]: lane holds m = col, k = 8*half .. 8*half+7
//                  B[k][n]: lane holds n = col, k = 8*half .. 8*half+7
//                  C[m][n]: lane holds n = col, m = 8*(v/4) + 4*half + v%4,
//                           v = 0..15
//   32x32x2 f32    A: m = col, k = half;  B: n = col, k = half;  C as above.
// A contraction index may be permuted freely as long as A and B agree; both
// operands below are built with the same (half, element) -> index map.
//
// K/V tiles are double-buffered in LDS: while a tile is consumed from one
// buffer, the next tile -- possibly the first tile of the next ring round --
// is fetched from HBM into registers and written to the other buffer, so
// the stream continues across round boundaries without a drain.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "ra_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup

struct KVBlock {
  const void* k;       // [B, len, H, D]
  const void* v;       // [B, len, H, D]
  long long k_pos0;    // global position of key row 0
  int len;             // rows in the block
  int cls;             // RA_FULL or RA_DIAG (SKIP blocks are not passed)
};

struct AttnArgs {
  const void* q;       // [B, Sq, H, D]
  void* o;             // [B, Sq, H, D]: fp32 if o_fp32, else the input dtype
  float* lse;          // [B, Sq, H] or null
  float* m_out;        // [B, Sq, H] or null
  float* l_out;        // [B, Sq, H] or null
  long long q_pos0;
  long long valid_len; // keys at global positions >= valid_len are padding
  int B, Sq, H;
  int n_qtiles;
  int causal;
  int o_fp32;
  float scale_log2;    // scale * log2(e): scores live in the base-2 domain
  int nblk;
  KVBlock blk[RA_MAX_P];
};

constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a per-lane value with the one held by lane l ^ 32 (the other half
// of the wave) through v_permlane32_swap.  After the swap, one of the two
// results is this lane's own value and the other its partner's, so max and
// sum over the pair need not know which is which.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Number of K/V tiles of block `b` this workgroup must visit: all tiles up
// to the last one holding a visible key ([RA] §3.4 applied per tile: tiles
// wholly in the future of the workgroup's last query, or wholly padding,
// are never read).
template <int BC>
__device__ __forceinline__ int tiles_of(const AttnArgs& a, int b, long long q_hi) {
  const KVBlock& kb = a.blk[b];
  const int n = (kb.len + BC - 1) / BC;
  long long lim = a.valid_len - 1;
  if (a.causal && q_hi < lim) lim = q_hi;
  if (lim < kb.k_pos0) return 0;
  const long long last = (lim - kb.k_pos0) / BC + 1;
  return last < n ? (int)last : n;
}

// Workgroup -> (batch, head, query tile).  Workgroups are dispatched
// round-robin over the 8 XCDs; the remap gives every XCD a contiguous range
// of tiles so the workgroups resident on one XCD share the same heads' K/V in
// that XCD's L2.  Within a head, later query tiles (more causal work) go
// first.
__device__ __forceinline__ void tile_coords(const AttnArgs& a, int& b, int& h, int& qt) {
  const int n = gridDim.x;
  int id = blockIdx.x;
  if ((n & 7) == 0) id = (id & 7) * (n >> 3) + (id >> 3);
  qt = id % a.n_qtiles;
  const int bh = id / a.n_qtiles;
  h = bh % a.H;
  b = bh / a.H;
  qt = a.n_qtiles - 1 - qt;
}

// Shared per-row bookkeeping of the online softmax for one lane (one query
// column, one half of the keys of every tile).
struct RowState {
  float m;   // running max of the scaled scores (base 2), -inf before any key
  float l;   // this lane's half of the running denominator
};

// Apply the recurrence of [RA] §3.2 to the NS raw scores of this lane:
//   m' = max(m, scale * max s), alpha = 2^(m - m'), p = 2^(scale*s - m'),
//   l' = alpha l + sum p; returns alpha (the caller rescales u).
template <int NS>
__device__ __forceinline__ float online_update(float (&s)[NS], RowState& st, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) mx = fmaxf(mx, s[i]);
  mx = pair_max(mx);
  const float m_new = fmaxf(st.m, mx * c);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    s[i] = fast_exp2(fmaf(s[i], c, -m_use));
    sum += s[i];
  }
  st.l = fmaf(alpha, st.l, sum);
  st.m = m_new;
  return alpha;
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
template <int D>
struct Bf16Cfg {
  static constexpr int BC = 64;                 // keys per tile
  static constexpr int KS = D * 2 + 16;         // K row stride in LDS (bytes)
  static constexpr int VS = BC * 2 + 16;        // V^T row stride in LDS (bytes)
  static constexpr int K_BYTES = BC * KS;
  static constexpr int V_BYTES = D * VS;
  static constexpr int BUF = K_BYTES + V_BYTES;
  static constexpr int K_UNITS = BC * D / 8 / kThreads;     // 16B per unit
  static constexpr int V_ITEMS = (BC / 4) * (D / 8);        // 4 keys x 8 d
  static constexpr int V_PER_T = (V_ITEMS + kThreads - 1) / kThreads;
  static constexpr int NC = D / 16;                         // k-steps of QK^T
  static constexpr int NDT = D / 32;                        // d tiles of O^T
};

// Position of key `g*4` (a group of 4 keys) inside the permuted V^T row:
// within each 16-key group the four 4-key groups are stored in the order
// 0, 2, 1, 3, so that lane half h reads its 8 keys {4h..4h+3, 8+4h..8+4h+3}
// as one 16-byte load.
__device__ __forceinline__ int vt_key_slot(int g) {
  const int G = g >> 2, gg = g & 3;
  const int pg = (gg == 1) ? 2 : (gg == 2 ? 1 : gg);
  return G * 16 + pg * 4;
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16(const AttnArgs a) {
  using C = Bf16Cfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  int b, h, qt;
  tile_coords(a, b, h, qt);
  const int row0 = qt * kBR;                       // first local row of the WG
  const int rows_here = min(kBR, a.Sq - row0);
  const long long q_lo = a.q_pos0 + row0;
  const long long q_hi = q_lo + rows_here - 1;
  const int wrow0 = row0 + wave * 32;              // first row of this wave
  const int wrows = min(32, a.Sq - wrow0);         // may be <= 0
  const long long wq_lo = a.q_pos0 + wrow0;
  const long long wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;         // row stride (elements)

  // Q fragment (B operand of S^T = K Q^T): query row wrow0+col,
  // features 16c + 8*half .. +7.
  bf16x8 qf[C::NC];
  {
    const int r = wrow0 + col;
    const __bf16* qp = (const __bf16*)a.q + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      if (r < a.Sq) qf[c] = *(const bf16x8*)(qp + 16 * c + 8 * half);
      else qf[c] = bf16x8{};
    }
  }

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) oacc[i] = f32x16{};
  RowState st{-INFINITY, 0.0f};

  // ---- tile cursor over (block, tile) in ring order ----
  int cb = 0, ct = 0, cn = 0;
  while (cb < a.nblk && (cn = tiles_of<BC>(a, cb, q_hi)) == 0) ++cb;
  bool have = cb < a.nblk;

  uint4 kreg[C::K_UNITS];
  uint4 vreg[C::V_PER_T][4];

  auto fetch = [&](int bi, int ti) {
    const KVBlock& kb = a.blk[bi];
    const int kt0 = ti * BC;
    const __bf16* kp = (const __bf16*)kb.k + ((long long)b * kb.len + kt0) * HD + (long long)h * D;
    const __bf16* vp = (const __bf16*)kb.v + ((long long)b * kb.len + kt0) * HD + (long long)h * D;
    const int rows = min(BC, kb.len - kt0);
#pragma unroll
    for (int u = 0; u < C::K_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int r = unit / (D / 8), c = unit % (D / 8);
      kreg[u] = r < rows ? *(const uint4*)(kp + r * HD + 8 * c) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int item = tid + u * kThreads;
      const int g = item % (BC / 4), c = item / (BC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        vreg[u][e] = (item < C::V_ITEMS && r < rows)
                         ? *(const uint4*)(vp + r * HD + 8 * c) : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_lds = [&](int buf) {
    char* kl = smem + buf * C::BUF;
    char* vl = kl + C::K_BYTES;
#pragma unroll
    for (int u = 0; u < C::K_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int r = unit / (D / 8), c = unit % (D / 8);
      *(uint4*)(kl + r * C::KS + 16 * c) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int item = tid + u * kThreads;
      if (item < C::V_ITEMS) {
        const int g = item % (BC / 4), c = item / (BC / 4);
        const int slot = vt_key_slot(g);
        const unsigned* w0 = (const unsigned*)&vreg[u][0];
        const unsigned* w1 = (const unsigned*)&vreg[u][1];
        const unsigned* w2 = (const unsigned*)&vreg[u][2];
        const unsigned* w3 = (const unsigned*)&vreg[u][3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const int sh = (e & 1) * 16;
          const unsigned lo = ((w0[w] >> sh) & 0xffffu) | (((w1[w] >> sh) & 0xffffu) << 16);
          const unsigned hi = ((w2[w] >> sh) & 0xffffu) | (((w3[w] >> sh) & 0xffffu) << 16);
          *(uint2*)(vl + (8 * c + e) * C::VS + slot * 2) = uint2{lo, hi};
        }
      }
    }
  };

  const float c_scale = a.scale_log2;
  int buf = 0;
  if (have) {
    fetch(cb, ct);
    store_lds(0);
  }
  __syncthreads();

  while (have) {
    // advance the cursor: next tile of this block, or the first tile of the
    // next visited block in ring order
    int nb = cb, nt = ct + 1, nn = cn;
    if (nt >= nn) {
      nt = 0;
      ++nb;
      while (nb < a.nblk && (nn = tiles_of<BC>(a, nb, q_hi)) == 0) ++nb;
    }
    const bool has_next = nb < a.nblk;
    if (has_next) fetch(nb, nt);

    // ---- compute on the current tile ----
    const KVBlock& kb = a.blk[cb];
    const int kt0 = ct * BC;
    const long long kp0 = kb.k_pos0 + kt0;
    const bool wave_live = wrows > 0 && !(a.causal && kp0 > wq_hi);
    if (wave_live) {
      const char* kl = smem + buf * C::BUF;
      const char* vl = kl + C::K_BYTES;
      float s[BC / 2];  // 2 S^T tiles x 16 values
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int c = 0; c < C::NC; ++c) {
          const bf16x8 kf = *(const bf16x8*)(kl + (32 * kt + col) * C::KS + (16 * c + 8 * half) * 2);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kt * 16 + v] = acc[v];
      }
      const bool need_mask =
          kt0 + BC > kb.len ||
          (kb.cls == RA_DIAG &&
           (kp0 + BC - 1 >= a.valid_len || (a.causal && kp0 + BC - 1 > wq_lo)));
      if (need_mask) {
        const long long qpos = wq_lo + col;
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
            const long long kpos = kp0 + j;
            const bool masked = kt0 + j >= kb.len || kpos >= a.valid_len ||
                                (a.causal && kpos > qpos);
            if (masked) s[kt * 16 + v] = -INFINITY;
          }
      }
      const float alpha = online_update<BC / 2>(s, st, c_scale);
#pragma unroll
      for (int i = 0; i < C::NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      // P^T in bf16: for key group G (16 keys), the lane's 8 values
      bf16x8 pb[BC / 16];
#pragma unroll
      for (int G = 0; G < BC / 16; ++G)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[G][e] = (__bf16)s[(G >> 1) * 16 + (G & 1) * 8 + e];
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int G = 0; G < BC / 16; ++G) {
          const bf16x8 vf = *(const bf16x8*)(vl + (32 * dt + col) * C::VS + (16 * G + 8 * half) * 2);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[G], oacc[dt], 0, 0, 0);
        }
    }

    if (has_next) store_lds(buf ^ 1);
    __syncthreads();
    cb = nb;
    ct = nt;
    cn = nn;
    have = has_next;
    buf ^= 1;
  }

  // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int r = wrow0 + col;
  if (wrows > 0 && r < a.Sq) {
    const long long ro = ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const float x0 = oacc[dt][4 * g + 0] * inv, x1 = oacc[dt][4 * g + 1] * inv;
        const float x2 = oacc[dt][4 * g + 2] * inv, x3 = oacc[dt][4 * g + 3] * inv;
        if (a.o_fp32) {
          *(float4*)((float*)a.o + ro + d) = float4{x0, x1, x2, x3};
        } else {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 y;
          y[0] = (__bf16)x0; y[1] = (__bf16)x1; y[2] = (__bf16)x2; y[3] = (__bf16)x3;
          *(bf16x4*)((__bf16*)a.o + ro + d) = y;
        }
      }
    if (half == 0) {
      const long long so = ((long long)b * a.Sq + r) * a.H + h;
      const bool seen = l_tot > 0.0f;
      if (a.lse) a.lse[so] = seen ? (st.m + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (a.m_out) a.m_out[so] = seen ? st.m * kLn2 : -INFINITY;
      if (a.l_out) a.l_out[so] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (no bf16 rounding anywhere; fp32 matrix-core products)
// ---------------------------------------------------------------------------
template <int D>
struct F32Cfg {
  static constexpr int BC = 32;
  static constexpr int KS = D * 4 + 16;  // K row stride (bytes)
  static constexpr int VS = D * 4 + 16;  // V row stride (bytes)
  static constexpr int K_BYTES = BC * KS;
  static constexpr int BUF = K_BYTES + BC * VS;
  static constexpr int UNITS = BC * D / 4 / kThreads;  // 16B units per thread
  static constexpr int NC4 = D / 8;                    // float4 steps of QK^T
  static constexpr int NDT = D / 32;
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_f32(const AttnArgs a) {
  using C = F32Cfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  int b, h, qt;
  tile_coords(a, b, h, qt);
  const int row0 = qt * kBR;
  const int rows_here = min(kBR, a.Sq - row0);
  const long long q_lo = a.q_pos0 + row0;
  const long long q_hi = q_lo + rows_here - 1;
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = a.q_pos0 + wrow0;
  const long long wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;

  // Q fragment: feature index of (step c4, element e) for this half is
  // 8*c4 + 4*half + e (the same map is used for K).
  float4 qf[C::NC4];
  {
    const int r = wrow0 + col;
    const float* qp = (const float*)a.q + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int c = 0; c < C::NC4; ++c)
      qf[c] = r < a.Sq ? *(const float4*)(qp + 8 * c + 4 * half) : float4{0, 0, 0, 0};
  }

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) oacc[i] = f32x16{};
  RowState st{-INFINITY, 0.0f};

  int cb = 0, ct = 0, cn = 0;
  while (cb < a.nblk && (cn = tiles_of<BC>(a, cb, q_hi)) == 0) ++cb;
  bool have = cb < a.nblk;

  float4 kreg[C::UNITS], vreg[C::UNITS];
  auto fetch = [&](int bi, int ti) {
    const KVBlock& kb = a.blk[bi];
    const int kt0 = ti * BC;
    const float* kp = (const float*)kb.k + ((long long)b * kb.len + kt0) * HD + (long long)h * D;
    const float* vp = (const float*)kb.v + ((long long)b * kb.len + kt0) * HD + (long long)h * D;
    const int rows = min(BC, kb.len - kt0);
#pragma unroll
    for (int u = 0; u < C::UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int r = unit / (D / 4), c = unit % (D / 4);
      kreg[u] = r < rows ? *(const float4*)(kp + r * HD + 4 * c) : float4{0, 0, 0, 0};
      vreg[u] = r < rows ? *(const float4*)(vp + r * HD + 4 * c) : float4{0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int buf) {
    char* kl = smem + buf * C::BUF;
    char* vl = kl + C::K_BYTES;
#pragma unroll
    for (int u = 0; u < C::UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int r = unit / (D / 4), c = unit % (D / 4);
      *(float4*)(kl + r * C::KS + 16 * c) = kreg[u];
      *(float4*)(vl + r * C::VS + 16 * c) = vreg[u];
    }
  };

  const float c_scale = a.scale_log2;
  int buf = 0;
  if (have) {
    fetch(cb, ct);
    store_lds(0);
  }
  __syncthreads();

  while (have) {
    int nb = cb, nt = ct + 1, nn = cn;
    if (nt >= nn) {
      nt = 0;
      ++nb;
      while (nb < a.nblk && (nn = tiles_of<BC>(a, nb, q_hi)) == 0) ++nb;
    }
    const bool has_next = nb < a.nblk;
    if (has_next) fetch(nb, nt);

    const KVBlock& kb = a.blk[cb];
    const int kt0 = ct * BC;
    const long long kp0 = kb.k_pos0 + kt0;
    const bool wave_live = wrows > 0 && !(a.causal && kp0 > wq_hi);
    if (wave_live) {
      const char* kl = smem + buf * C::BUF;
      const char* vl = kl + C::K_BYTES;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NC4; ++c) {
        const float4 kf = *(const float4*)(kl + col * C::KS + (8 * c + 4 * half) * 4);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qf[c].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qf[c].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qf[c].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qf[c].w, acc, 0, 0, 0);
      }
      float s[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = acc[v];
      const bool need_mask =
          kt0 + BC > kb.len ||
          (kb.cls == RA_DIAG &&
           (kp0 + BC - 1 >= a.valid_len || (a.causal && kp0 + BC - 1 > wq_lo)));
      if (need_mask) {
        const long long qpos = wq_lo + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 8 * (v >> 2) + 4 * half + (v & 3);
          const long long kpos = kp0 + j;
          if (kt0 + j >= kb.len || kpos >= a.valid_len || (a.causal && kpos > qpos))
            s[v] = -INFINITY;
        }
      }
      const float alpha = online_update<16>(s, st, c_scale);
#pragma unroll
      for (int i = 0; i < C::NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      // O^T += V^T P^T; k index of step v for this half = the score's key
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 8 * (v >> 2) + 4 * half + (v & 3);
          const float vf = *(const float*)(vl + j * C::VS + (32 * dt + col) * 4);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, s[v], oacc[dt], 0, 0, 0);
        }
    }

    if (has_next) store_lds(buf ^ 1);
    __syncthreads();
    cb = nb;
    ct = nt;
    cn = nn;
    have = has_next;
    buf ^= 1;
  }

  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int r = wrow0 + col;
  if (wrows > 0 && r < a.Sq) {
    const long long ro = ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        *(float4*)((float*)a.o + ro + d) =
            float4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                   oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
      }
    if (half == 0) {
      const long long so = ((long long)b * a.Sq + r) * a.H + h;
      const bool seen = l_tot > 0.0f;
      if (a.lse) a.lse[so] = seen ? (st.m + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (a.m_out) a.m_out[so] = seen ? st.m * kLn2 : -INFINITY;
      if (a.l_out) a.l_out[so] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
ra_status launch(const AttnArgs& a, int D, ra_dtype dt, hipStream_t stream,
                 const char* name) {
  const long long n_wg = (long long)a.B * a.H * a.n_qtiles;
  if (n_wg == 0) return RA_OK;
  if (n_wg > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: too many query tiles", name);
  const dim3 grid((unsigned)n_wg), block(kThreads);
  if (dt == RA_BF16) {
    if (D == 128) hipLaunchKernelGGL(ring_attn_bf16<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(ring_attn_bf16<64>, grid, block, 0, stream, a);
  } else {
    if (D == 128) hipLaunchKernelGGL(ring_attn_f32<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(ring_attn_f32<64>, grid, block, 0, stream, a);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}

ra_status check_common(const char* name, int B, int S, int H, int D, ra_dtype dt) {
  if (B < 0 || S < 0 || H < 0)
    return ra::fail(RA_ERR_SHAPE, "%s: negative size (B=%d S=%d H=%d)", name, B, S, H);
  if (dt != RA_BF16 && dt != RA_FP32)
    return ra::fail(RA_ERR_DTYPE, "%s: unknown dtype %d", name, (int)dt);
  if (D != 64 && D != 128)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: head dimension %d not supported "
                    "(64 or 128)", name, D);
  return RA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" ra_status ra_block_attn_fwd(const void* q, const void* k, const void* v,
                                       int B, int Sq, int Sk, int H, int D,
                                       ra_dtype dt, float scale, long long q_pos0,
                                       long long k_pos0, int causal,
                                       long long valid_len, float* o, float* lse,
                                       float* m_opt, float* l_opt, void* stream) {
  static const char* name = "ra_block_attn_fwd";
  ra::clear_error();
  ra_status st = check_common(name, B, Sq, H, D, dt);
  if (st != RA_OK) return st;
  if (Sk < 0) return ra::fail(RA_ERR_SHAPE, "%s: negative Sk", name);
  const long long n_out = (long long)B * Sq * H;
  if (n_out == 0) return RA_OK;
  if (!q || !o || !lse || (Sk > 0 && (!k || !v)))
    return ra::fail(RA_ERR_NULL, "%s: NULL q/k/v/o/lse", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return ra::fail(RA_ERR_SHAPE, "%s: q, k, v and o must be 16-byte aligned", name);
  if (q_pos0 < 0 || k_pos0 < 0)
    return ra::fail(RA_ERR_RANGE, "%s: negative global position", name);
  if (valid_len < 0) valid_len = INT64_MAX;
  AttnArgs a{};
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.m_out = m_opt;
  a.l_out = l_opt;
  a.q_pos0 = q_pos0;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
  a.n_qtiles = (Sq + kBR - 1) / kBR;
  a.causal = causal != 0;
  a.o_fp32 = 1;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.nblk = 0;
  const int cls = ra::block_class(q_pos0, q_pos0 + Sq, k_pos0, k_pos0 + Sk,
                                  a.causal, valid_len);
  if (cls != RA_SKIP) {
    a.blk[0] = KVBlock{k, v, k_pos0, Sk, cls};
    a.nblk = 1;
  }
  return launch(a, D, dt, (hipStream_t)stream, name);
}

extern "C" ra_status ra_ring_attn_fwd(const void* q_r, const void* const* k_blocks,
                                      const void* const* v_blocks, int B, int Sb,
                                      int H, int D, int P, int rank, ra_dtype dt,
                                      float scale, int causal, long long valid_len,
                                      void* o, float* lse_opt, void* stream) {
  static const char* name = "ra_ring_attn_fwd";
  ra::clear_error();
  ra_status st = check_common(name, B, Sb, H, D, dt);
  if (st != RA_OK) return st;
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (P > RA_MAX_P)
    return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P=%d", name, P, RA_MAX_P);
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  const long long n_out = (long long)B * Sb * H;
  if (n_out == 0) return RA_OK;
  if (!q_r || !o || !k_blocks || !v_blocks)
    return ra::fail(RA_ERR_NULL, "%s: NULL q/o/block table", name);
  if (!aligned16(q_r) || !aligned16(o))
    return ra::fail(RA_ERR_SHAPE, "%s: q and o must be 16-byte aligned", name);
  const long long S = (long long)P * Sb;
  if (valid_len < 0 || valid_len > S) valid_len = S;
  AttnArgs a{};
  a.q = q_r;
  a.o = o;
  a.lse = lse_opt;
  a.q_pos0 = (long long)rank * Sb;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sb;
  a.H = H;
  a.n_qtiles = (Sb + kBR - 1) / kBR;
  a.causal = causal != 0;
  a.o_fp32 = dt == RA_FP32;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  // the ring schedule of [RA] §3.3 with the block classes of §3.4; SKIP
  // blocks are dropped here and never read by the kernel
  int src[RA_MAX_P], cls[RA_MAX_P];
  st = ra_ring_schedule(P, rank, Sb, causal, valid_len, src, cls);
  if (st != RA_OK) return st;
  a.nblk = 0;
  for (int t = 0; t < P; ++t) {
    if (cls[t] == RA_SKIP) continue;
    const int j = src[t];
    if (!k_blocks[j] || !v_blocks[j])
      return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited block %d", name, j);
    if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]))
      return ra::fail(RA_ERR_SHAPE, "%s: block %d not 16-byte aligned", name, j);
    a.blk[a.nblk++] = KVBlock{k_blocks[j], v_blocks[j], (long long)j * Sb, Sb, cls[t]};
  }
  return launch(a, D, dt, (hipStream_t)stream, name);
}
