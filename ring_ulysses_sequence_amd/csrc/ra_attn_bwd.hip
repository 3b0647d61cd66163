// Backward of ring-order block attention on CDNA4 (gfx950).
//
// What is computed ([RA] §3.3 closing paragraph, §6.2): rank r holds Q_r,
// the upstream gradient dO_r, and the forward's output O_r and natural
// log-sum-exp lse_r.  For every visited K/V block j (ring order, future
// blocks skipped when causal) it recomputes the block's probabilities from
// the saved statistics, P_j = exp(scale * Q_r K_j^T - lse_r) (masked pairs
// 0), and with D_r = rowsum(dO_r * O_r):
//   dV_j += P_j^T dO_r
//   dS_j  = P_j * (dO_r V_j^T - D_r)
//   dQ_r += scale * dS_j K_j
//   dK_j += scale * dS_j^T Q_r
// dK_j and dV_j are the parts that belong to block j's owner (the ring sums
// them over all query shards); dQ_r is complete after all blocks.
//
// Two kernels, bf16 operands and fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_bf16; the operand layouts are those of the forward
// kernels: A[m][k] lane holds m = col, k = 8*half ..; B[k][n] lane holds
// n = col, k = 8*half ..; C[m][n] lane holds n = col, m = 8*(v/4) + 4*half +
// v%4):
//   ring_attn_bwd_dq<D>:  one workgroup per 128 query rows (4 waves x 32).
//     Each lane holds one query column: S^T = K Q^T and dP^T = V dO^T from
//     K/V rows in LDS, then dQ^T += K^T dS^T with K^T read transposed
//     (ds_read_b64_tr_b16) and dS^T from registers -- the forward's P V step
//     with V replaced by K.  It also writes D_r for the second kernel.
//   ring_attn_bwd_dkv<D, PART>: one workgroup per 128 keys of one visited
//     block (4 waves x 32 keys).  Each lane holds one key column: S = Q K^T
//     (and, for dK, dP = dO V^T) from Q/dO rows in LDS, then dV^T += dO^T P
//     (PART 0) or dK^T += Q^T dS (PART 1) with dO^T / Q^T read transposed.
//     Two launches rather than one so that each fits two waves per SIMD.
// Tiles (64 rows) are staged through registers: the next tile's global
// loads are issued before the current tile is computed and written to the
// other LDS buffer after it, one barrier per tile.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "ra_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows (dq) or keys (dkv) per workgroup
constexpr int kTile = 64;           // rows per staged tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdBlock {
  const void* k;      // [B, kv_rows_b, H, D] bf16, this block's rows from 0
  const void* v;
  float* dk;          // [B, kv_rows_b, H, D] fp32, accumulated (+=)
  float* dv;
  long long k_pos0;   // global position of key row 0
  int len;            // rows in the block
  int pad;
};

struct BwdArgs {
  const void* q;      // [B, Sq, H, D] bf16
  const void* o;      // [B, Sq, H, D] bf16
  const void* dout;   // [B, Sq, H, D] bf16
  const float* lse;   // [B, Sq, H] natural log-sum-exp of the forward
  float* dq;          // [B, Sq, H, D] fp32, accumulated (+=)
  float* delta;       // [B, Sq, H] fp32: rowsum(dO * O), written by the dq kernel
  long long q_pos0;   // global position of query row 0
  long long valid_len;
  int B, Sq, H;
  int kv_rows_b;      // rows between consecutive batches in every K/V buffer
  int causal;
  int n_ktiles;       // 128-key tiles per block (dkv grid)
  float scale;
  float scale_log2;
  int nblk;
  BwdBlock blk[RA_MAX_P];
};

template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  // 16-byte chunk c of row r: XOR swizzle that spreads a column of rows over
  // the LDS banks (the forward's K layout)
  return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ s16x4 read_tr(const char* smem, unsigned off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(smem + off));
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  const s16x4 x[2] = {lo, hi};
  bf16x8 r;
  __builtin_memcpy(&r, x, 16);
  return r;
}

// A 64-row tile of a [B, rows_b, H, D] bf16 tensor staged through registers
// into LDS (swizzled rows of D*2 bytes).  Each thread moves UNITS chunks of
// 16 bytes; rows at or beyond `rows` read as zeros.
template <int D>
struct TileStage {
  static constexpr int ROWB = D * 2;
  static constexpr int BYTES = kTile * ROWB;
  static constexpr int CHUNKS = D / 8;
  static constexpr int UNITS = BYTES / 16 / kThreads;
  u32x4 r[UNITS];
  __device__ __forceinline__ void load(const char* base, int rows, long long row_stride) {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int p = i * kThreads + (int)threadIdx.x;
      const int row = p / CHUNKS, c = p % CHUNKS;
      r[i] = row < rows ? *(const u32x4*)(base + row * row_stride + c * 16) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int p = i * kThreads + (int)threadIdx.x;
      const int row = p / CHUNKS, c = p % CHUNKS;
      *(u32x4*)(lds + row * ROWB + swz<D>(row, c) * 16) = r[i];
    }
  }
};

// Per-lane LDS byte offsets of the operand reads inside one staged tile:
//   row_off[c]: A/B fragment of row `col`, features 16c + 8*half .. +7
//   tr_lo[dt], tr_hi[dt]: transposed reads of rows 4*half + e (+8 for hi) at
//   features 32*dt + 16*(g & 1) + 4*q (ds_read_b64_tr_b16: lane j of each
//   16-lane group receives element j%4 of the rows supplied by lanes j/4 +
//   4e, so lane l ends with features 32*dt + l%32 of 4 consecutive rows)
template <int D>
struct TileAddr {
  static constexpr int ROWB = D * 2;
  static constexpr int NC = D / 16;
  static constexpr int NDT = D / 32;
  int row_off[NC];
  unsigned tr_lo[NDT], tr_hi[NDT];
  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c = 0; c < NC; ++c) row_off[c] = col * ROWB + swz<D>(col, 2 * c + half) * 16;
    const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
    const int kl = 4 * half + e;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
      tr_lo[dt] = kl * ROWB + swz<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
      tr_hi[dt] = (kl + 8) * ROWB + swz<D>(kl + 8, d0 >> 3) * 16 + (d0 & 7) * 2;
    }
  }
  // transposed A fragment of feature tile dt over rows 16G .. 16G+15
  __device__ __forceinline__ bf16x8 tr(const char* tile, int G, int dt) const {
    return join(read_tr(tile, tr_lo[dt] + 16 * G * ROWB), read_tr(tile, tr_hi[dt] + 16 * G * ROWB));
  }
  __device__ __forceinline__ bf16x8 row(const char* tile, int rt, int c) const {
    return *(const bf16x8*)(tile + rt * 32 * ROWB + row_off[c]);
  }
};

// ---------------------------------------------------------------------------
// dQ (and D = rowsum(dO * O)): one workgroup per (batch, head, 128 rows)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bwd_dq(const BwdArgs a) {
  constexpr int NC = D / 16, NDT = D / 32, ROWB = D * 2;
  using TS = TileStage<D>;
  // two buffers, each a K tile then a V tile
  __shared__ __attribute__((aligned(16))) char smem[2][2 * TS::BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int n_qt = (a.Sq + kRows - 1) / kRows;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = qt * kRows;
  const long long q_hi = a.q_pos0 + min(row0 + kRows, a.Sq) - 1;
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = a.q_pos0 + wrow0, wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;
  const long long row_stride = HD * 2;  // bytes between K/V rows

  // this lane's query row: Q and dO fragments (B operands), D and lse
  const int r = wrow0 + col;
  const bool row_ok = r < a.Sq;
  bf16x8 qf[NC], df[NC];
  float dsum = 0.0f;
  {
    const long long off = ((long long)b * a.Sq + r) * HD + (long long)h * D;
    const __bf16* qp = (const __bf16*)a.q + off;
    const __bf16* dp = (const __bf16*)a.dout + off;
    const __bf16* op = (const __bf16*)a.o + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d = 16 * c + 8 * half;
      qf[c] = row_ok ? *(const bf16x8*)(qp + d) : bf16x8{};
      df[c] = row_ok ? *(const bf16x8*)(dp + d) : bf16x8{};
      const bf16x8 of = row_ok ? *(const bf16x8*)(op + d) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)df[c][e] * (float)of[e];
    }
  }
  dsum = pair_sum(dsum);
  const long long so = ((long long)b * a.Sq + r) * a.H + h;
  if (row_ok && half == 0) a.delta[so] = dsum;
  // base-2 lse; a row that saw no key in the forward gets +inf, so every
  // probability of it is 0 (its scores are all masked anyway)
  float lse2 = INFINITY;
  if (row_ok) {
    const float l = a.lse[so];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
  }

  TileAddr<D> ad;
  ad.init(lane);
  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16{};

  // visited tiles: all blocks in order, tiles up to the last one with a
  // key visible to the workgroup's last query
  auto ntiles = [&](int bi) -> int {
    const BwdBlock& kb = a.blk[bi];
    const int n = (kb.len + kTile - 1) / kTile;
    long long lim = a.valid_len - 1;
    if (a.causal && q_hi < lim) lim = q_hi;
    if (lim < kb.k_pos0) return 0;
    const long long last = (lim - kb.k_pos0) / kTile + 1;
    return last < n ? (int)last : n;
  };
  int cb = 0, ct = 0, cn = 0;
  while (cb < a.nblk && (cn = ntiles(cb)) == 0) ++cb;

  // one staging register set, used for the next tile's K, then its V
  TS st;
  auto src_of = [&](int bi, int ti, const void* base) -> const char* {
    return (const char*)base +
           (((long long)b * a.kv_rows_b + (long long)ti * kTile) * a.H + h) * D * 2;
  };
  int buf = 0;
  if (cb < a.nblk) {
    const int rows = min(kTile, a.blk[cb].len);
    st.load(src_of(cb, 0, a.blk[cb].k), rows, row_stride);
    st.store(smem[0]);
    st.load(src_of(cb, 0, a.blk[cb].v), rows, row_stride);
    st.store(smem[0] + TS::BYTES);
  }
  __syncthreads();
  const float c_scale = a.scale_log2;
  while (cb < a.nblk) {
    // next tile's position; its K loads fly during the first half of this
    // tile, its V loads during the second (the other buffer was last read
    // in the previous iteration, before its closing barrier)
    int nb = cb, nt = ct + 1, nn = cn;
    if (nt >= nn) {
      nt = 0;
      ++nb;
      while (nb < a.nblk && (nn = ntiles(nb)) == 0) ++nb;
    }
    const bool more = nb < a.nblk;
    const int nrows = more ? min(kTile, a.blk[nb].len - nt * kTile) : 0;
    if (more) st.load(src_of(nb, nt, a.blk[nb].k), nrows, row_stride);

    const BwdBlock& kb = a.blk[cb];
    const long long kp0 = kb.k_pos0 + (long long)ct * kTile;
    const char* kt = smem[buf];
    const char* vt = smem[buf] + TS::BYTES;
    const bool live = wrows > 0 && !(a.causal && kp0 > wq_hi);
    // mask: key j of the tile (j = 32t + 8(v/4) + 4half + v%4) is hidden
    // for this lane's query when j >= the keys left in the block or at or
    // beyond valid_len, or (causal) when it lies after the query
    long long lim_ll = kb.len - (long long)ct * kTile;
    if (a.valid_len - kp0 < lim_ll) lim_ll = a.valid_len - kp0;
    const bool need = lim_ll < kTile || (a.causal && kp0 + kTile - 1 > wq_lo);
    long long lim = lim_ll;
    if (a.causal) {
      const long long rel = wq_lo + col - kp0 + 1;  // keys 0 .. rel-1 visible
      if (rel < lim) lim = rel;
    }
    // as a 32-bit bound relative to this lane's first key of each group
    const int lim_h = (int)(lim < 0 ? 0 : (lim > kTile ? kTile : lim)) - 4 * half;
    // one 32-key half of the tile at a time (keeps two waves per SIMD)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (live) {
        f32x16 sc = f32x16{}, dpt = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.row(kt, t, c), qf[c], sc, 0, 0, 0);
          dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.row(vt, t, c), df[c], dpt, 0, 0, 0);
          // keep the operand reads next to their products (bounded live range)
          __builtin_amdgcn_sched_barrier(0);
        }
        if (need) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * t + 8 * (v >> 2) + (v & 3) >= lim_h) sc[v] = -INFINITY;
        }
        // dS^T = P^T (dP^T - D), packed as the B operand of K^T dS^T
        bf16x8 dsb[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(sc[v] * c_scale - lse2);
          dsb[v >> 3][v & 7] = (__bf16)(p * (dpt[v] - dsum));
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.tr(kt, 2 * t + g, dt), dsb[g],
                                                              acc[dt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if (t == 0 && more) {
        st.store(smem[buf ^ 1]);
        st.load(src_of(nb, nt, a.blk[nb].v), nrows, row_stride);
      }
    }
    if (more) st.store(smem[buf ^ 1] + TS::BYTES);
    __syncthreads();
    buf ^= 1;
    cb = nb;
    ct = nt;
    cn = nn;
  }

  // dQ += scale * (dS K): this lane's row, features 32dt + 8g + 4half .. +3
  if (row_ok) {
    float* dqp = a.dq + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4* p = (float4*)(dqp + 32 * dt + 8 * g + 4 * half);
        float4 x = *p;
        x.x += a.scale * acc[dt][4 * g + 0];
        x.y += a.scale * acc[dt][4 * g + 1];
        x.z += a.scale * acc[dt][4 * g + 2];
        x.w += a.scale * acc[dt][4 * g + 3];
        *p = x;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (visited block, batch, head, 128 keys)
// ---------------------------------------------------------------------------
// PART 0 accumulates dV (needs S only), PART 1 dK (needs S and dP): split so
// that each fits two waves per SIMD; the scores are recomputed in both.
template <int D, int PART>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bwd_dkv(const BwdArgs a) {
  constexpr int NC = D / 16, NDT = D / 32;
  using TS = TileStage<D>;
  // two buffers, each: Q tile, dO tile, lse2 (64 floats), D (64 floats)
  constexpr int BUF = 2 * TS::BYTES + 2 * kTile * 4;
  __shared__ __attribute__((aligned(16))) char smem[2][BUF];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  int id = blockIdx.x;
  const int kt = id % a.n_ktiles;
  id /= a.n_ktiles;
  const int h = id % a.H;
  id /= a.H;
  const int b = id % a.B;
  const int bi = id / a.B;
  const BwdBlock& kb = a.blk[bi];
  const long long HD = (long long)a.H * D;
  const long long row_stride = HD * 2;

  // this lane's key row of the block: K and V fragments (B operands)
  const int kr = kt * kRows + wave * 32 + col;
  const bool key_ok = kr < kb.len;
  const long long kpos = kb.k_pos0 + kr;
  const long long kw_lo = kb.k_pos0 + kt * kRows + wave * 32;
  const long long kw_hi = kw_lo + 31;
  constexpr bool DK = PART == 1;
  bf16x8 kf[NC], vf[DK ? NC : 1];
  {
    const long long off = ((long long)b * a.kv_rows_b + kr) * HD + (long long)h * D;
    const __bf16* kp = (const __bf16*)kb.k + off;
    const __bf16* vp = (const __bf16*)kb.v + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d = 16 * c + 8 * half;
      kf[c] = key_ok ? *(const bf16x8*)(kp + d) : bf16x8{};
      if constexpr (DK) vf[c] = key_ok ? *(const bf16x8*)(vp + d) : bf16x8{};
    }
  }
  TileAddr<D> ad;
  ad.init(lane);
  f32x16 acc[NDT];  // dK^T (PART 1) or dV^T (PART 0)
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x16{};

  // query tiles that can see a key of this workgroup (causal: from the one
  // holding position k_lo on)
  const long long k_lo = kb.k_pos0 + (long long)kt * kRows;
  int t0 = 0;
  if (a.causal && k_lo > a.q_pos0) t0 = (int)min((long long)a.Sq, (k_lo - a.q_pos0) / kTile);
  const int n_t = (a.Sq + kTile - 1) / kTile;

  // one staging register set, used for the next tile's Q, then its dO
  TS st;
  float stat = 0.0f;  // one lse2 (threads 0-63) or D (64-127) value
  auto src_of = [&](int ti, const void* base) -> const char* {
    return (const char*)base + (((long long)b * a.Sq + (long long)ti * kTile) * a.H + h) * D * 2;
  };
  auto load_stat = [&](int ti) {
    if (tid < 2 * kTile) {
      const int rr = ti * kTile + (tid & (kTile - 1));
      const long long so = ((long long)b * a.Sq + rr) * a.H + h;
      if (tid < kTile) {
        // base-2 lse; +inf for rows past the end or rows that saw no key
        const float l = rr < a.Sq ? a.lse[so] : -INFINITY;
        stat = l == -INFINITY ? INFINITY : l * kLog2e;
      } else {
        stat = rr < a.Sq ? a.delta[so] : 0.0f;
      }
    }
  };
  auto put_stat = [&](char* dst) {
    if (tid < 2 * kTile) ((float*)(dst + 2 * TS::BYTES))[tid] = stat;
  };
  int buf = 0;
  if (t0 < n_t) {
    const int rows = min(kTile, a.Sq - t0 * kTile);
    st.load(src_of(t0, a.q), rows, row_stride);
    st.store(smem[0]);
    st.load(src_of(t0, a.dout), rows, row_stride);
    st.store(smem[0] + TS::BYTES);
    load_stat(t0);
    put_stat(smem[0]);
  }
  __syncthreads();
  const float c_scale = a.scale_log2;
  for (int ti = t0; ti < n_t; ++ti) {
    // next tile: its Q loads fly during the first half of this tile, its dO
    // loads during the second (the other buffer was last read in the
    // previous iteration, before its closing barrier)
    const bool more = ti + 1 < n_t;
    const int nrows = more ? min(kTile, a.Sq - (ti + 1) * kTile) : 0;
    if (more) {
      st.load(src_of(ti + 1, a.q), nrows, row_stride);
      load_stat(ti + 1);
    }
    const char* qt = smem[buf];
    const char* dt_ = smem[buf] + TS::BYTES;
    const float* ls = (const float*)(smem[buf] + 2 * TS::BYTES);
    const float* ds_ = ls + kTile;
    const long long qp0 = a.q_pos0 + (long long)ti * kTile;
    const long long qp_hi = qp0 + min(kTile, a.Sq - ti * kTile) - 1;
    const bool live = !(a.causal && kw_lo > qp_hi) && kw_lo < a.valid_len;
    // element (query m = 32t + 8g + 4half + i of the tile, this lane's key)
    // is hidden when the key is padding or (causal) after the query, i.e.
    // m < rel with rel = key - first query of the tile (32-bit, clamped)
    const bool need = kw_hi >= a.valid_len || (a.causal && kw_hi > qp0);
    int rel = 0;
    if (kpos >= a.valid_len) rel = kTile;
    else if (a.causal) rel = (int)max(0LL, min((long long)kTile, kpos - qp0));
    const int rel_h = rel - 4 * half;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (live) {
        f32x16 sc = f32x16{}, dpt = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.row(qt, t, c), kf[c], sc, 0, 0, 0);
          if constexpr (DK)
            dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.row(dt_, t, c), vf[c], dpt, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m0 = 32 * t + 8 * g + 4 * half;
          const float4 l4 = *(const float4*)(ls + m0);
          const float4 d4 = *(const float4*)(ds_ + m0);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 4 * g + i;
            float x = sc[v] * c_scale - lv[i];
            if (need && 32 * t + 8 * g + i < rel_h) x = -INFINITY;
            const float p = __builtin_amdgcn_exp2f(x);
            if constexpr (DK) sb[v >> 3][v & 7] = (__bf16)(p * (dpt[v] - dv4[i]));
            else pb[v >> 3][v & 7] = (__bf16)p;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int d = 0; d < NDT; ++d) {
            if constexpr (DK)
              acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.tr(qt, 2 * t + g, d), sb[g],
                                                               acc[d], 0, 0, 0);
            else
              acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.tr(dt_, 2 * t + g, d), pb[g],
                                                               acc[d], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      if (t == 0 && more) {
        st.store(smem[buf ^ 1]);
        st.load(src_of(ti + 1, a.dout), nrows, row_stride);
      }
    }
    if (more) {
      st.store(smem[buf ^ 1] + TS::BYTES);
      put_stat(smem[buf ^ 1]);
    }
    __syncthreads();
    buf ^= 1;
  }

  if (key_ok) {
    const long long off = ((long long)b * a.kv_rows_b + kr) * HD + (long long)h * D;
    float* dst = (DK ? kb.dk : kb.dv) + off;
    const float f = DK ? a.scale : 1.0f;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4* p = (float4*)(dst + 32 * d + 8 * g + 4 * half);
        float4 x = *p;
        x.x += f * acc[d][4 * g + 0];
        x.y += f * acc[d][4 * g + 1];
        x.z += f * acc[d][4 * g + 2];
        x.w += f * acc[d][4 * g + 3];
        *p = x;
      }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" ra_status ra_ring_attn_bwd(const void* q_r, const void* const* k_blocks,
                                      const void* const* v_blocks, const void* o_r,
                                      const void* do_r, const float* lse_r, int B, int Sb,
                                      int H, int D, int P, int rank, ra_dtype dt, float scale,
                                      int causal, long long valid_len, float* dq_r,
                                      float* const* dk_blocks, float* const* dv_blocks,
                                      float* delta_ws, void* stream) {
  static const char* name = "ra_ring_attn_bwd";
  ra::clear_error();
  if (B < 0 || Sb < 0 || H < 0)
    return ra::fail(RA_ERR_SHAPE, "%s: negative size (B=%d Sb=%d H=%d)", name, B, Sb, H);
  if (dt != RA_BF16 && dt != RA_FP32) return ra::fail(RA_ERR_DTYPE, "%s: unknown dtype %d", name, (int)dt);
  if (dt != RA_BF16) return ra::fail(RA_ERR_UNSUPPORTED, "%s: only bf16 inputs are supported", name);
  if (D != 64 && D != 128)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: head dimension %d not supported (64 or 128)", name, D);
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (P > RA_MAX_P) return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P=%d", name, P, RA_MAX_P);
  if (rank < 0 || rank >= P) return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  if ((long long)B * Sb * H == 0) return RA_OK;
  if (!q_r || !o_r || !do_r || !lse_r || !dq_r || !delta_ws || !k_blocks || !v_blocks ||
      !dk_blocks || !dv_blocks)
    return ra::fail(RA_ERR_NULL, "%s: NULL argument", name);
  if (!aligned16(q_r) || !aligned16(o_r) || !aligned16(do_r) || !aligned16(dq_r))
    return ra::fail(RA_ERR_SHAPE, "%s: q, o, do and dq must be 16-byte aligned", name);
  const long long S = (long long)P * Sb;
  if (valid_len < 0 || valid_len > S) valid_len = S;
  BwdArgs a{};
  a.q = q_r;
  a.o = o_r;
  a.dout = do_r;
  a.lse = lse_r;
  a.dq = dq_r;
  a.delta = delta_ws;
  a.q_pos0 = (long long)rank * Sb;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sb;
  a.H = H;
  a.kv_rows_b = Sb;
  a.causal = causal != 0;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale = (float)sc;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  // the ring schedule of [RA] §3.3 with the classes of §3.4; SKIP blocks
  // are neither read nor written
  int src[RA_MAX_P], cls[RA_MAX_P];
  ra_status st = ra_ring_schedule(P, rank, Sb, causal, valid_len, src, cls);
  if (st != RA_OK) return st;
  a.nblk = 0;
  for (int t = 0; t < P; ++t) {
    if (cls[t] == RA_SKIP) continue;
    const int j = src[t];
    if (!k_blocks[j] || !v_blocks[j] || !dk_blocks[j] || !dv_blocks[j])
      return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited block %d", name, j);
    if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]) || !aligned16(dk_blocks[j]) ||
        !aligned16(dv_blocks[j]))
      return ra::fail(RA_ERR_SHAPE, "%s: block %d not 16-byte aligned", name, j);
    a.blk[a.nblk++] = BwdBlock{k_blocks[j], v_blocks[j], dk_blocks[j], dv_blocks[j],
                               (long long)j * Sb, Sb, 0};
  }
  hipStream_t s = (hipStream_t)stream;
  const long long n_dq = (long long)B * H * ((Sb + kRows - 1) / kRows);
  a.n_ktiles = (Sb + kRows - 1) / kRows;
  const long long n_dkv = (long long)a.nblk * B * H * a.n_ktiles;
  if (n_dq > 0x7fffffffLL || n_dkv > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: grid too large", name);
  // dq first: it writes D = rowsum(dO * O), which the dk/dv kernel reads
  if (D == 128) hipLaunchKernelGGL(ring_attn_bwd_dq<128>, dim3((unsigned)n_dq), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(ring_attn_bwd_dq<64>, dim3((unsigned)n_dq), dim3(kThreads), 0, s, a);
  if (n_dkv > 0) {
    const dim3 g((unsigned)n_dkv);
    if (D == 128) {
      hipLaunchKernelGGL((ring_attn_bwd_dkv<128, 0>), g, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((ring_attn_bwd_dkv<128, 1>), g, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((ring_attn_bwd_dkv<64, 0>), g, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((ring_attn_bwd_dkv<64, 1>), g, dim3(kThreads), 0, s, a);
    }
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}
