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
//   ring_attn_bwd_dq<D, NW>: one workgroup per 32*NW query rows (NW = 8
//     waves when that still fills the compute units, else 4).  Each lane
//     holds one query column: S^T = K Q^T and dP^T = V dO^T from
//     K/V rows in LDS, then dQ^T += K^T dS^T with K^T read transposed
//     (ds_read_b64_tr_b16) and dS^T from registers -- the forward's P V step
//     with V replaced by K.  It also writes the per-row statistics the second
//     kernel reads: the base-2 lse and D_r.
//   ring_attn_bwd_dkv_pair<D>: one workgroup per 128 keys of one visited
//     block, 8 waves: each lane holds one key column, and the two waves of a
//     SIMD split the work on their 32 keys -- one computes S = Q K^T, P and
//     dV^T += dO^T P, the other dP = dO V^T, dS = P (dP - D) with its
//     partner's P (handed over in LDS) and dK^T += Q^T dS, with dO^T / Q^T
//     read transposed.  (One wave doing both would not fit in 256 registers;
//     two separate launches would compute S and P twice.)
// Tiles of 64 rows are copied HBM -> LDS by the buffer unit (buffer_load ...
// lds).  The dQ kernel double-buffers: the copy of tile n+1 is issued when
// tile n starts and has the whole of tile n's compute to land; one wait and
// one barrier per tile.  The dK/dV kernel keeps three buffers and runs in
// half-tile steps with one barrier each (see pair_body).  Every tile is read
// both ways -- by rows (ds_read_b128, 16 lanes a pass: rows 0..15 at one
// chunk) and transposed (ds_read_b64_tr_b16, 32 lanes a pass: rows 4k..4k+3
// at four adjacent chunks 4t..4t+3) -- so rows are stored with an XOR swizzle
// of their 16-byte chunks that keeps both free of bank conflicts (64 banks of
// 4 bytes): chunk c of row r sits at c ^ h(r) with
//   D = 128: h(r) = (r & 3) << 2 | (r >> 2) & 3
//            (a permutation of 0..15 over any 16 rows, and the four rows of
//            an aligned group of 4 fall into four different chunk groups)
//   D = 64:  with s = (r >> 1) & 7, h(r) = (s & 1) << 2 | s >> 1
//            (two rows share a 256-byte bank line; the same two properties
//            for the rows of one parity)
// The copy picks for every LDS position the global chunk that belongs there.
// Operand reads run kPF matrix-op pairs ahead of their use.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "ra_cdna4.h"
#include "ra_internal.h"
#include "ra_order.h"

namespace {

using namespace ra_cdna4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 128;          // keys per dK/dV workgroup (4 wave pairs x 32)
constexpr int kTile = 64;           // rows per copied tile
constexpr int kPF = 2;              // operand reads in flight ahead of use (pairs)
constexpr float kLog2e = 1.4426950408889634f;

struct BwdBlock {
  const void* k;      // [B, kv_rows_b, Hkv, D] bf16, this block's rows from 0
  const void* v;
  float* dk;          // [B, kv_rows_b, Hkv, D] fp32, accumulated (+=)
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
  float* stats;       // [2, B, H, Sq] fp32: base-2 lse, then -rowsum(dO * O);
                      // written by the dq kernel, read by the dk/dv kernel
  long long q_pos0;   // global position of query row 0
  // query row r sits at q_pos0 + r below q_split, at q_pos1 + (r - q_split)
  // from it on (the two chunks of a zigzag share; q_split is a multiple of
  // 64 and positions increase with the row)
  long long q_pos1;
  int q_split;
  long long valid_len;
  int B, Sq, H;
  int Hkv;            // K/V heads (H % Hkv == 0): query head h uses K/V head
                      // h / (H / Hkv); dK/dV sum over the query heads of a group
  int kv_rows_b;      // rows between consecutive batches in every K/V buffer
  int causal;
  int n_ktiles;       // 128-key tiles per block (dkv grid)
  float scale;
  float scale_log2;
  // rotation of the block table for the later query tiles of the lockstep
  // order of ra_order.h, 0 for none: 1 when every key of the blocks after
  // the first is visible to every query, 2 for a causal zigzag share (its
  // own two chunks first); used by the 8-wave dq kernel
  int lockstep;
  int nblk;
  BwdBlock blk[RA_MAX_P];
};

__device__ __forceinline__ long long qpos(const BwdArgs& a, int row) {
  return row < a.q_split ? a.q_pos0 + row : a.q_pos1 + (row - a.q_split);
}

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;                   // bytes per row in LDS
  static constexpr int TILE = kTile * ROWB;            // one copied tile
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
  static constexpr int NC = D / 16;                    // k-steps of the score products
  static constexpr int NDT = D / 32;                   // 32-feature tiles of the gradients
};

template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  const int s = (r >> 1) & 7;
  return c ^ (((s & 1) << 2) | (s >> 1));
}

__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 as_bf16(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f32x4 as_f32(u32x4 x) { return __builtin_bit_cast(f32x4, x); }

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  const s16x4 x[2] = {lo, hi};
  bf16x8 r;
  __builtin_memcpy(&r, x, 16);
  return r;
}

// Copy one 64-row tile (rows at or beyond `rows` read as zeros) whose row 0
// starts at `src`, rows HD2 bytes apart, into LDS, shared by NWV waves: this
// wave's TILE / 1024 / NWV KiB land at byte address dst, dst + 1024, ..;
// voff[i] is the source offset of this lane's chunk (row * HD2 + swizzled
// chunk * 16).
template <int D, int NWV>
__device__ __forceinline__ void copy_tile(const char* src, int rows, int HD2, const int* voff,
                                          unsigned dst) {
  using C = Cfg<D>;
  constexpr int DMA = C::TILE / 1024 / NWV;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src, 0, (rows - 1) * HD2 + C::ROWB, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < DMA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(size_t)(dst + i * 1024), 16,
                                             voff[i], 0, 0, 0);
}

// Per-lane LDS byte addresses of the operand reads in the current buffer:
//   row[c]: A fragment of row `col`, features 16c + 8*half .. +7
//   lo[dt], hi[dt]: transposed reads of rows 4*half + e (+8 for hi) at
//   features 32*dt + 16*(g & 1) + 4*q (ds_read_b64_tr_b16: lane j of each
//   16-lane group receives element j%4 of the rows supplied by lanes j/4 +
//   4e, so lane l ends with features 32*dt + l%32 of 4 consecutive rows)
// Rows 32t + col (row reads) and 16G + .. (transposed reads) keep the same
// swizzle, so those tiles are reached through the immediate offset.
template <int D>
struct LaneAddr {
  using C = Cfg<D>;
  unsigned row[C::NC], lo[C::NDT], hi[C::NDT];
  __device__ __forceinline__ void init(unsigned base, int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) row[c] = base + col * C::ROWB + swz<D>(col, 2 * c + half) * 16;
    const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
    const int kl = 4 * half + e;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
      lo[dt] = base + kl * C::ROWB + swz<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
      hi[dt] = base + (kl + 8) * C::ROWB + swz<D>(kl + 8, d0 >> 3) * 16 + (d0 & 7) * 2;
    }
  }
};

// Transposed read of rows 16G + .. (G = 2T + g, g a constant after unrolling)
// at tile offset OFF.
template <int D, int OFF>
__device__ __forceinline__ s16x4 read_tr_g(int g, unsigned addr) {
  constexpr int G1 = 16 * Cfg<D>::ROWB;
  return g ? lds_read_tr16<OFF + G1>(addr) : lds_read_tr16<OFF>(addr);
}

// Source offsets of this lane's copy chunks within a tile copied by NWV
// waves.
template <int D, int NWV>
__device__ __forceinline__ void copy_offsets(int wave, int lane, int HD2, int* voff) {
  using C = Cfg<D>;
  constexpr int DMA = C::TILE / 1024 / NWV;
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int p = (wave * DMA + i) * 64 + lane;  // physical chunk in the tile
    const int r = p / C::CHUNKS, pc = p % C::CHUNKS;
    voff[i] = r * HD2 + swz<D>(r, pc) * 16;
  }
}

// ---------------------------------------------------------------------------
// dQ (and the row statistics): one workgroup per (batch, head, 128 rows)
// ---------------------------------------------------------------------------
template <int D>
struct DqLane {
  using C = Cfg<D>;
  bf16x8 qf[C::NC], df[C::NC];  // this lane's query row of Q and dO (B operands)
  f32x16 acc[C::NDT];           // dQ^T
  f32x16 negd;                  // -D of this lane's query in every element: the
                                // dP^T accumulators start from it, so they end
                                // holding dP - D
  LaneAddr<D> ad;
};

// Rows 32T .. 32T+31 of the K/V tiles in the buffer at byte offset BO from
// buffer 0 (K at BO, V at BO + TILE): S^T, dP^T, the mask, dS^T and
// dQ^T += K^T dS^T.
struct NoWork {
  __device__ void operator()() const {}
};
// after_first: scalar work (the next tile's copy) issued once the first
// matrix ops are under way.
template <int D, int T, int BO, class Hook = NoWork>
__device__ __forceinline__ void dq_half(DqLane<D>& w, float dsum, float lse2, float c_scale,
                                        bool need, int lim_h,
                                        const Hook& after_first = Hook{}) {
  using C = Cfg<D>;
  constexpr int RO = BO + T * 32 * C::ROWB;
  constexpr int NB = kPF + 1;
  f32x16 sc = f32x16{}, dpt = w.negd;
  {
    u32x4 ka[NB], va[NB];
#pragma unroll
    for (int c = 0; c < kPF; ++c) {
      ka[c] = lds_read_b128<RO>(w.ad.row[c]);
      va[c] = lds_read_b128<C::TILE + RO>(w.ad.row[c]);
    }
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      if (c + kPF < C::NC) {
        ka[(c + kPF) % NB] = lds_read_b128<RO>(w.ad.row[c + kPF]);
        va[(c + kPF) % NB] = lds_read_b128<C::TILE + RO>(w.ad.row[c + kPF]);
      }
      const int n = 2 * min(kPF, C::NC - 1 - c);
      claim_lds_n(n, ka[c % NB]);
      claim_lds_n(n, va[c % NB]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(ka[c % NB]), w.qf[c], sc, 0, 0, 0);
      dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(va[c % NB]), w.df[c], dpt, 0, 0, 0);
      if (c == 0) after_first();
    }
  }
  // the first K^T reads of the dQ product fly during the exponentials
  constexpr int NJ = 2 * C::NDT;  // (g, dt) pairs, g major
  s16x4 lo[NB], hi[NB];
#pragma unroll
  for (int j = 0; j < kPF; ++j) {
    lo[j] = read_tr_g<D, BO + 32 * T * C::ROWB>(j / C::NDT, w.ad.lo[j % C::NDT]);
    hi[j] = read_tr_g<D, BO + 32 * T * C::ROWB>(j / C::NDT, w.ad.hi[j % C::NDT]);
  }
  // key j of the tile (j = 32T + 8(v/4) + 4half + v%4) is hidden for this
  // lane's query when j >= lim_h + 4half
  if (need) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (32 * T + 8 * (v >> 2) + (v & 3) >= lim_h) sc[v] = -INFINITY;
  }
  // dS^T = P^T (dP^T - D), packed as the B operand of K^T dS^T
  bf16x8 dsb[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float p = __builtin_amdgcn_exp2f(sc[v] * c_scale - lse2);
    dsb[v >> 3][v & 7] = (__bf16)(p * dpt[v]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j + kPF < NJ) {
      const int jn = j + kPF;
      lo[jn % NB] = read_tr_g<D, BO + 32 * T * C::ROWB>(jn / C::NDT, w.ad.lo[jn % C::NDT]);
      hi[jn % NB] = read_tr_g<D, BO + 32 * T * C::ROWB>(jn / C::NDT, w.ad.hi[jn % C::NDT]);
    }
    const int n = 2 * min(kPF, NJ - 1 - j);
    claim_lds_n(n, lo[j % NB]);
    claim_lds_n(n, hi[j % NB]);
    const int dt = j % C::NDT;
    w.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(lo[j % NB], hi[j % NB]),
                                                        dsb[j / C::NDT], w.acc[dt], 0, 0, 0);
  }
}

// NW waves of 32 query rows share each K/V tile in LDS: 8 (one workgroup
// per compute unit, half the K/V streamed per query row) when that still
// gives every compute unit a workgroup, else 4 (two per compute unit).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bwd_dq(const BwdArgs a) {
  using C = Cfg<D>;
  constexpr int ROWS = 32 * NW;                 // query rows per workgroup
  constexpr int DMA = C::TILE / 1024 / NW;      // 1 KiB copies per wave per tile
  // two buffers, each a K tile then a V tile
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * C::TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 31,
            half = lane >> 5;
  const int n_qt = (a.Sq + ROWS - 1) / ROWS;
  // Workgroups are dispatched round-robin over the 8 XCDs: remap so that
  // every XCD takes a contiguous range of heads, and the workgroups resident
  // on it (neighbouring query tiles of one head) stream the same K/V tiles
  // through its L2; later query tiles (more causal work) first.  With 8
  // waves, the lockstep order of ra_order.h where it applies.
  int bh, qt, rot = 0;
  if (NW != 8 || !a.lockstep || a.nblk <= 0 ||
      !ra_order::lockstep_coords((int)blockIdx.x, (int)gridDim.x, n_qt, a.B * a.H,
                                 a.lockstep % a.nblk, bh, qt, rot)) {
    int id = blockIdx.x;
    if ((gridDim.x & 7) == 0) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
    bh = id / n_qt;
    qt = n_qt - 1 - id % n_qt;
  }
  const int b = bh / a.H, h = bh % a.H;
  const int row0 = qt * ROWS;
  const long long q_hi = qpos(a, min(row0 + ROWS, a.Sq) - 1);
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = qpos(a, wrow0), wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;
  const int hk = h / (a.H / a.Hkv);            // K/V head of this query head
  const int HD2 = a.Hkv * D * 2;               // bytes between K/V rows

  // this lane's query row: Q and dO fragments, D and the base-2 lse
  DqLane<D> w;
  const int r = wrow0 + col;
  const bool row_ok = r < a.Sq;
  float dsum = 0.0f;
  {
    const long long off = ((long long)b * a.Sq + r) * HD + (long long)h * D;
    const __bf16* qp = (const __bf16*)a.q + off;
    const __bf16* dp = (const __bf16*)a.dout + off;
    const __bf16* op = (const __bf16*)a.o + off;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const int d = 16 * c + 8 * half;
      w.qf[c] = row_ok ? *(const bf16x8*)(qp + d) : bf16x8{};
      w.df[c] = row_ok ? *(const bf16x8*)(dp + d) : bf16x8{};
      const bf16x8 of = row_ok ? *(const bf16x8*)(op + d) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)w.df[c][e] * (float)of[e];
    }
  }
  dsum = pair_sum(dsum);
  // a row that saw no key in the forward gets +inf, so every probability of
  // it is 0 (its scores are all masked anyway); so does a padding query
  // (position >= valid_len): padding rows are discarded, not part of the
  // loss, and with P = 0 and D = 0 none of their terms reaches dq, dk or dv
  // whatever dO holds there
  float lse2 = INFINITY;
  const bool row_real = row_ok && qpos(a, r) < a.valid_len;
  if (!row_real) dsum = 0.0f;
  if (row_ok) {
    const float l = a.lse[((long long)b * a.Sq + r) * a.H + h];
    lse2 = l == -INFINITY || !row_real ? INFINITY : l * kLog2e;
    if (half == 0) {
      const long long so = ((long long)b * a.H + h) * a.Sq + r;
      a.stats[so] = lse2;
      a.stats[(long long)a.B * a.H * a.Sq + so] = -dsum;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) w.acc[i] = f32x16{};
#pragma unroll
  for (int v = 0; v < 16; ++v) w.negd[v] = -dsum;
  const unsigned base = lds_addr(smem);
  w.ad.init(base, lane);
  int voff[DMA];
  copy_offsets<D, NW>(wave, lane, HD2, voff);
  const unsigned dst0 = base + wave * DMA * 1024;

  // visited tiles: all blocks in order from table entry rot on (wrapping
  // around), tiles up to the last one with a key visible to the workgroup's
  // last query; cb / nb below count blocks in that order
  auto entry = [&](int p) -> int {
    const int i = p + rot;
    return i >= a.nblk ? i - a.nblk : i;
  };
  auto ntiles = [&](int p) -> int {
    const BwdBlock& kb = a.blk[entry(p)];
    const int n = (kb.len + kTile - 1) / kTile;
    long long lim = a.valid_len - 1;
    if (a.causal && q_hi < lim) lim = q_hi;
    if (lim < kb.k_pos0) return 0;
    const long long last = (lim - kb.k_pos0) / kTile + 1;
    return last < n ? (int)last : n;
  };
  auto copy_kv = [&](int p, int ti, unsigned dst) {
    const BwdBlock& kb = a.blk[entry(p)];
    const long long off =
        (((long long)b * a.kv_rows_b + (long long)ti * kTile) * a.Hkv + hk) * D * 2;
    const int rows = min(kTile, kb.len - ti * kTile);
    copy_tile<D, NW>((const char*)kb.k + off, rows, HD2, voff, dst);
    copy_tile<D, NW>((const char*)kb.v + off, rows, HD2, voff, dst + C::TILE);
  };
  int cb = 0, ct = 0, cn = 0;
  while (cb < a.nblk && (cn = ntiles(cb)) == 0) ++cb;
  if (cb < a.nblk) copy_kv(cb, 0, dst0);
  wait_vmcnt<0>();
  pipeline_barrier();
  const float c_scale = a.scale_log2;
  // one tile from the buffer at byte offset BO (0 or 2 TILE); the loop below
  // alternates the two, so that every operand read carries its buffer
  // offset as an immediate
  auto step = [&](auto boc) {
    constexpr int BO = decltype(boc)::value;
    // the next tile's copy goes to the other buffer, last read in the
    // previous step (before its closing barrier)
    int nb = cb, nt = ct + 1, nn = cn;
    if (nt >= nn) {
      nt = 0;
      ++nb;
      while (nb < a.nblk && (nn = ntiles(nb)) == 0) ++nb;
    }
    // issued from the first matrix ops of the tile (the target buffer was
    // released by the barrier that ended the previous step)
    auto copies = [&]() {
      if (nb < a.nblk) copy_kv(nb, nt, dst0 + (BO ? 0 : 2 * C::TILE));
    };

    const BwdBlock& kb = a.blk[entry(cb)];
    const long long kp0 = kb.k_pos0 + (long long)ct * kTile;
    const bool live = wrows > 0 && !(a.causal && kp0 > wq_hi);
    // mask: key j of the tile is hidden for this lane's query when j >= the
    // keys left in the block or at or beyond valid_len, or (causal) when it
    // lies after the query
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
    if (live) {
      dq_half<D, 0, BO>(w, dsum, lse2, c_scale, need, lim_h, copies);
      dq_half<D, 1, BO>(w, dsum, lse2, c_scale, need, lim_h);
    } else {
      copies();
    }
    wait_vmcnt<0>();
    pipeline_barrier();
    cb = nb;
    ct = nt;
    cn = nn;
  };
  while (cb < a.nblk) {
    step(std::integral_constant<int, 0>{});
    if (cb >= a.nblk) break;
    step(std::integral_constant<int, 2 * C::TILE>{});
  }

  // dQ += scale * (dS K): this lane's row, features 32dt + 8g + 4half .. +3
  if (row_ok) {
    float* dqp = a.dq + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4* p = (float4*)(dqp + 32 * dt + 8 * g + 4 * half);
        float4 x = *p;
        x.x += a.scale * w.acc[dt][4 * g + 0];
        x.y += a.scale * w.acc[dt][4 * g + 1];
        x.z += a.scale * w.acc[dt][4 * g + 2];
        x.w += a.scale * w.acc[dt][4 * g + 3];
        *p = x;
      }
  }
}

// ---------------------------------------------------------------------------
// dK and dV together: one workgroup of 8 waves per (visited block, batch,
// head, 128 keys).  Waves g and g + 4 run on one SIMD and share the 32 keys
// of group g:
//   role 0 (wave g):     S = Q K^T, P = exp(S - lse) (masked), P to LDS,
//                        dV^T += dO^T P
//   role 1 (wave g + 4): dP = dO V^T; after the barrier, dS = P (dP - D)
//                        with its partner's P, dK^T += Q^T dS
// so the scores and exponentials are computed once per key, not once per
// gradient.  Both roles share the Q / dO tiles in LDS; each half tile (32
// query rows) has one barrier for the P hand-over, each tile one more for
// its copies.  Within a step each wave runs its two matrix chains as one
// stream of operand reads (the second chain's first reads fly during the
// first chain) with its element-wise work placed between matrix ops.
// ---------------------------------------------------------------------------
constexpr int kPairThreads = 512;
constexpr int kXSlot = 32 * 32 * 2;  // P of one key group for one half tile

template <int D>
struct PairCfg {
  static constexpr int BUF = 2 * Cfg<D>::TILE + 2 * kTile * 4;  // Q, dO, lse2, D
  static constexpr int NBUF = 3;                                // tiles it, it+1, it+2
  static constexpr int XB = NBUF * BUF;                         // P exchange
  static constexpr int LDS = XB + 2 * 4 * kXSlot;               // two half parities
  static constexpr int DMA = Cfg<D>::TILE / 1024 / 8;
};

template <int D, int ROLE>
struct PairLane {
  using C = Cfg<D>;
  bf16x8 f[C::NC];     // K (role 0) or V (role 1) row of this lane's key
  f32x16 acc[C::NDT];  // dV^T (role 0) or dK^T (role 1)
  LaneAddr<D> ad;
  unsigned sa;         // this lane's statistics in the current buffer
  unsigned xa;         // this lane's slot in the P exchange (parity 0)
};

// The LDS operand stream of one step: N1 row reads (one instruction each)
// for the first matrix chain, then N2 transposed pairs (two each) for the
// second, issued kPairLead operands ahead of their matrix ops across the
// boundary between the chains.  after(i): the LDS instructions issued after
// operand i's own when matrix op i waits for it.
constexpr int kPairLead = 2;

template <int N1, int N2>
struct OpStream {
  static constexpr int N = N1 + N2;
  static constexpr int cnt(int i) { return i < N1 ? 1 : 2; }
  static constexpr int after(int i) {
    int n = 0;
    for (int m = i + 1; m <= i + kPairLead && m < N; ++m) n += cnt(m);
    return n;
  }
};

// Role 0, one step.  F: the scores S^T = K Q^T of half TF (query rows
// 32TF .. 32TF+31) of the tile in buffer bof, and from them P (masked,
// rounded to bf16) into pf and into the lane's exchange slot.  B: dV^T +=
// dO^T P^T of half TB of the tile in buffer bob, with that half's P in pb.
// The exponentials of the new P run between the dV matrix ops.
template <int D, bool F, bool B, int TF, int TB>
__device__ __forceinline__ void step_p(PairLane<D, 0>& w, unsigned bof, unsigned bob, bool need,
                                       int rel_h, float c_scale, bf16x8 (&pf)[2],
                                       const bf16x8 (&pb)[2]) {
  using C = Cfg<D>;
  constexpr int N1 = F ? C::NC : 0, N2 = B ? 2 * C::NDT : 0;
  using S = OpStream<N1, N2>;
  constexpr int NB = kPairLead + 1;
  constexpr int AO = TF * 32 * C::ROWB;            // Q rows
  constexpr int TO = C::TILE + TB * 32 * C::ROWB;  // dO^T
  constexpr int SO = 2 * C::TILE + 128 * TF;       // lse2
  constexpr int XO = TF * 4 * kXSlot;
  constexpr int PV = 16 / (2 * C::NDT);            // P values per dV matrix op
  u32x4 ra[NB], st[4];
  s16x4 lo[NB], hi[NB];
  f32x16 sc = f32x16{};
  if constexpr (F) {
    const unsigned sa = w.sa + bof;
    st[0] = lds_read_b128<SO + 0>(sa);
    st[1] = lds_read_b128<SO + 32>(sa);
    st[2] = lds_read_b128<SO + 64>(sa);
    st[3] = lds_read_b128<SO + 96>(sa);
  }
  auto issue = [&](int i) {
    if (i < N1) {
      ra[i % NB] = lds_read_b128<AO>(w.ad.row[i] + bof);
    } else {
      const int j = i - N1;
      lo[i % NB] = read_tr_g<D, TO>(j / C::NDT, w.ad.lo[j % C::NDT] + bob);
      hi[i % NB] = read_tr_g<D, TO>(j / C::NDT, w.ad.hi[j % C::NDT] + bob);
    }
  };
  // P of (query m = 32TF + 8g + 4half + i, this lane's key) for v = 4g + i,
  // hidden when m < rel_h + 4half.  The mask goes into the statistics: on a
  // tile that needs it (a uniform branch, taken on diagonal, padded and
  // dead tiles only) the base-2 lse of every hidden query of the lane is
  // set to +inf, so its weight exp2(s - inf) is 0 and the weights themselves
  // take no test.
  auto mask_stats = [&]() {
    if (need) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int g = v >> 2, i = v & 3;
        if (32 * TF + 8 * g + i < rel_h) st[g][i] = __float_as_uint(INFINITY);
      }
    }
  };
  auto p_val = [&](int v) {
    const int g = v >> 2, i = v & 3;
    const float x = sc[v] * c_scale - as_f32(st[g])[i];
    pf[v >> 3][v & 7] = (__bf16)__builtin_amdgcn_exp2f(x);
  };
#pragma unroll
  for (int i = 0; i < kPairLead; ++i)
    if (i < S::N) issue(i);
#pragma unroll
  for (int i = 0; i < S::N; ++i) {
    if (i + kPairLead < S::N) issue(i + kPairLead);
    const int n = S::after(i);
    if (i < N1) {
      claim_lds_n(n, ra[i % NB]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(ra[i % NB]), w.f[i], sc, 0, 0, 0);
    } else {
      const int j = i - N1;
      claim_lds_n(n, lo[i % NB]);
      claim_lds_n(n, hi[i % NB]);
      if (F && j == 0) {
        // the statistics were read before every operand
        claim_lds_n(n, st[0]);
        claim_lds_n(n, st[1]);
        claim_lds_n(n, st[2]);
        claim_lds_n(n, st[3]);
        mask_stats();
      }
      w.acc[j % C::NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          join(lo[i % NB], hi[i % NB]), pb[j / C::NDT], w.acc[j % C::NDT], 0, 0, 0);
      if constexpr (F) {
#pragma unroll
        for (int e = 0; e < PV; ++e) p_val(PV * j + e);
      }
    }
  }
  if constexpr (F) {
    if constexpr (!B) {
      claim_lds<0>(st[0]);
      claim_lds<0>(st[1]);
      claim_lds<0>(st[2]);
      claim_lds<0>(st[3]);
      mask_stats();
#pragma unroll
      for (int v = 0; v < 16; ++v) p_val(v);
    }
    lds_write_b128<XO>(w.xa, __builtin_bit_cast(u32x4, pf[0]));
    lds_write_b128<XO + 1024>(w.xa, __builtin_bit_cast(u32x4, pf[1]));
  }
}

// Role 1, one step.  B: dS^T = P^T o (dP^T - D) of half TB from its dP in
// scb, its D in stb and the partner's P in the exchange (rounded to bf16),
// then dK^T += Q^T dS^T of that half (tile in buffer bob).  F: dP^T = V dO^T
// of half TF of the tile in buffer bof into scf, with that half's D into stf.
// dS is formed between the dP matrix ops.
template <int D, bool F, bool B, int TF, int TB>
__device__ __forceinline__ void step_ds(PairLane<D, 1>& w, unsigned bof, unsigned bob,
                                        f32x16& scf, u32x4 (&stf)[4], const f32x16& scb,
                                        u32x4 (&stb)[4]) {
  using C = Cfg<D>;
  constexpr int N1 = F ? C::NC : 0, N2 = B ? 2 * C::NDT : 0;
  using S = OpStream<N1, N2>;
  constexpr int NB = kPairLead + 1;
  constexpr int AO = C::TILE + TF * 32 * C::ROWB;        // dO rows
  constexpr int TO = TB * 32 * C::ROWB;                  // Q^T
  constexpr int SO = 2 * C::TILE + 4 * kTile + 128 * TF;  // D
  constexpr int XO = TB * 4 * kXSlot;
  constexpr int PV = 16 / C::NC;                         // dS values per dP matrix op
  u32x4 ra[NB], x0, x1;
  s16x4 lo[NB], hi[NB];
  bf16x8 ds[2];
  if constexpr (B) {
    x0 = lds_read_b128<XO>(w.xa);
    x1 = lds_read_b128<XO + 1024>(w.xa);
  }
  if constexpr (F) {
    const unsigned sa = w.sa + bof;
    stf[0] = lds_read_b128<SO + 0>(sa);
    stf[1] = lds_read_b128<SO + 32>(sa);
    stf[2] = lds_read_b128<SO + 64>(sa);
    stf[3] = lds_read_b128<SO + 96>(sa);
  }
  auto issue = [&](int i) {
    if (i < N1) {
      ra[i % NB] = lds_read_b128<AO>(w.ad.row[i] + bof);
    } else {
      const int j = i - N1;
      lo[i % NB] = read_tr_g<D, TO>(j / C::NDT, w.ad.lo[j % C::NDT] + bob);
      hi[i % NB] = read_tr_g<D, TO>(j / C::NDT, w.ad.hi[j % C::NDT] + bob);
    }
  };
  // scb already holds dP - D: the dP products of its half accumulated onto
  // that half's -D (the statistics row holds -D)
  auto ds_val = [&](int v) {
    const bf16x8 p8 = as_bf16(v < 8 ? x0 : x1);
    const float p = (float)p8[v & 7];
    ds[v >> 3][v & 7] = (__bf16)(p * scb[v]);
  };
  auto claim_b = [&](int n) {
    claim_lds_n(n, x0);
    claim_lds_n(n, x1);
  };
  if constexpr (B && !F) {
    claim_b(0);
#pragma unroll
    for (int v = 0; v < 16; ++v) ds_val(v);
  }
#pragma unroll
  for (int i = 0; i < kPairLead; ++i)
    if (i < S::N) issue(i);
#pragma unroll
  for (int i = 0; i < S::N; ++i) {
    if (i + kPairLead < S::N) issue(i + kPairLead);
    const int n = S::after(i);
    if (i < N1) {
      claim_lds_n(n, ra[i % NB]);
      // the exchange and the statistics were read before every operand
      if (B && i == 0) claim_b(n);
      if (i == 0) {
        // dP^T accumulates onto -D of its queries (in the MFMA output layout)
        claim_lds_n(n, stf[0]);
        claim_lds_n(n, stf[1]);
        claim_lds_n(n, stf[2]);
        claim_lds_n(n, stf[3]);
        scf = __builtin_bit_cast(f32x16, stf);
      }
      scf = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(ra[i % NB]), w.f[i], scf, 0, 0, 0);
      if constexpr (B) {
#pragma unroll
        for (int e = 0; e < PV; ++e) ds_val(PV * i + e);
      }
    } else {
      const int j = i - N1;
      claim_lds_n(n, lo[i % NB]);
      claim_lds_n(n, hi[i % NB]);
      w.acc[j % C::NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          join(lo[i % NB], hi[i % NB]), ds[j / C::NDT], w.acc[j % C::NDT], 0, 0, 0);
    }
  }
}

// One step of either role with the parts that are live: f (the front half,
// TF) and b (the back half, TB).
template <int D, int ROLE, int TF, int TB>
__device__ __forceinline__ void pair_step(PairLane<D, ROLE>& w, bool f, bool b, unsigned bof,
                                          unsigned bob, bool need, int rel_h, float c_scale,
                                          bf16x8 (&pf)[2], const bf16x8 (&pb)[2], f32x16& scf,
                                          u32x4 (&stf)[4], const f32x16& scb, u32x4 (&stb)[4]) {
  if constexpr (ROLE == 0) {
    if (f && b) step_p<D, true, true, TF, TB>(w, bof, bob, need, rel_h, c_scale, pf, pb);
    else if (f) step_p<D, true, false, TF, TB>(w, bof, bob, need, rel_h, c_scale, pf, pb);
    else if (b) step_p<D, false, true, TF, TB>(w, bof, bob, need, rel_h, c_scale, pf, pb);
  } else {
    if (f && b) step_ds<D, true, true, TF, TB>(w, bof, bob, scf, stf, scb, stb);
    else if (f) step_ds<D, true, false, TF, TB>(w, bof, bob, scf, stf, scb, stb);
    else if (b) step_ds<D, false, true, TF, TB>(w, bof, bob, scf, stf, scb, stb);
  }
}

// Both parts of a step of either role (the steady state).
template <int D, int ROLE, int TF, int TB>
__device__ __forceinline__ void step_both(PairLane<D, ROLE>& w, unsigned bof, unsigned bob,
                                          bool need, int rel_h, float c_scale, bf16x8 (&pf)[2],
                                          const bf16x8 (&pb)[2], f32x16& scf, u32x4 (&stf)[4],
                                          const f32x16& scb, u32x4 (&stb)[4]) {
  if constexpr (ROLE == 0) step_p<D, true, true, TF, TB>(w, bof, bob, need, rel_h, c_scale, pf, pb);
  else step_ds<D, true, true, TF, TB>(w, bof, bob, scf, stf, scb, stb);
}

template <int D, int ROLE>
__device__ __forceinline__ void pair_body(const BwdArgs& a, char* smem, int wave, int lane) {
  using C = Cfg<D>;
  using PC = PairCfg<D>;
  const int g = wave & 3, half = lane >> 5, col = lane & 31;
  // XCD-contiguous ranges as in the dQ kernel, over (batch, K/V head) major,
  // then visited block, then key tile: the workgroups resident on one XCD
  // are neighbouring key tiles of one block and head, which stream the same
  // Q / dO tiles through its L2, and every XCD's range spans all blocks (the
  // diagonal block's lighter work spread evenly)
  int id = blockIdx.x;
  if ((gridDim.x & 7) == 0) id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
  const int kt = id % a.n_ktiles;
  id /= a.n_ktiles;
  const int bi = id % a.nblk;
  id /= a.nblk;
  const int hk = id % a.Hkv;  // K/V head; its query heads are hk*G .. hk*G + G-1
  const int b = id / a.Hkv;
  const int G = a.H / a.Hkv;
  const BwdBlock& kb = a.blk[bi];
  if (kt * kRows >= kb.len) return;  // a shorter block: no key of it here (uniform)
  const long long HDkv = (long long)a.Hkv * D;
  const int HD2 = a.H * D * 2;  // bytes between Q / dO rows

  const int kr = kt * kRows + g * 32 + col;
  const bool key_ok = kr < kb.len;
  const long long kpos = kb.k_pos0 + kr;
  const long long kw_lo = kb.k_pos0 + kt * kRows + g * 32;
  const long long kw_hi = kw_lo + 31;
  PairLane<D, ROLE> w;
  {
    const long long off = ((long long)b * a.kv_rows_b + kr) * HDkv + (long long)hk * D;
    const __bf16* fp = (const __bf16*)(ROLE == 0 ? kb.k : kb.v) + off;
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
      w.f[c] = key_ok ? *(const bf16x8*)(fp + 16 * c + 8 * half) : bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) w.acc[i] = f32x16{};
  const unsigned base = lds_addr(smem);
  w.ad.init(base, lane);
  w.sa = base + 16 * half;
  w.xa = base + PC::XB + g * kXSlot + lane * 16;
  int voff[PC::DMA];
  copy_offsets<D, 8>(wave, lane, HD2, voff);

  const long long k_lo = kb.k_pos0 + (long long)kt * kRows;
  int t0 = 0;
  if (a.causal) {
    // the first 64-row query tile whose last query is at or after k_lo
    // (tiles never straddle the split)
    if (k_lo <= a.q_pos0 + a.q_split - 1)
      t0 = k_lo > a.q_pos0 ? (int)((k_lo - a.q_pos0) / kTile) : 0;
    else
      t0 = a.q_split / kTile + (k_lo > a.q_pos1 ? (int)min((long long)a.Sq, (k_lo - a.q_pos1) / kTile) : 0);
    if (t0 > (a.Sq + kTile - 1) / kTile) t0 = (a.Sq + kTile - 1) / kTile;
  }
  const int n_t = (a.Sq + kTile - 1) / kTile;
  // the query tiles t0 .. n_t-1 of each query head of the group in turn
  const int n_per = n_t - t0, n_it = G * n_per;
  // Q and dO tiles by all eight waves; the statistics rows by waves 0 (lse)
  // and 1 (D)
  // (query head, query tile) of an iteration, advanced by one per
  // iteration (no division in the loop)
  // The copy cursor also carries its tile's byte offset in Q / dO, its
  // offset in the statistics rows and the rows left in the head, advanced
  // by additions.
  struct ItCur {
    int h, ti;
    long long qoff, soff;
    int left;
  };
  const long long q_step = (long long)kTile * HD2;
  auto it_start = [&](int h) {
    return ItCur{h, t0, (((long long)b * a.Sq + (long long)t0 * kTile) * a.H + h) * D * 2,
                 ((long long)b * a.H + h) * a.Sq + (long long)t0 * kTile, a.Sq - t0 * kTile};
  };
  auto it_next = [&](ItCur& c) {
    if (++c.ti == n_t) {
      c = it_start(c.h + 1);
    } else {
      c.qoff += q_step;
      c.soff += kTile;
      c.left -= kTile;
    }
  };
  const long long stat_plane = wave ? (long long)a.B * a.H * a.Sq : 0;
  auto copy_q = [&](const ItCur& c, unsigned buf_base) {
    const long long off = c.qoff;
    const int rows = min(kTile, c.left);
    const unsigned dst = buf_base + wave * PC::DMA * 1024;
    copy_tile<D, 8>((const char*)a.q + off, rows, HD2, voff, dst);
    copy_tile<D, 8>((const char*)a.dout + off, rows, HD2, voff, dst + C::TILE);
    if (wave < 2) {
      const float* src = a.stats + stat_plane + c.soff;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, rows * 4, kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void_ptr)(size_t)(buf_base + 2 * C::TILE + wave * 4 * kTile), 4, lane * 4, 0,
          0, 0);
    }
  };
  // Tile it sits in buffer it % 3.  The loop runs in half steps: between
  // barriers, role 0 forms the scores of the next half and then its dV
  // product of the current one, with the next half's P computed between the
  // dV matrix ops; role 1 forms the dP of the next half, with the current
  // half's dS computed between those matrix ops, and then its dK product of
  // the current half.  P of a half crosses over at the barrier that ends the
  // step forming it.  Tile it+2 is copied from the
  // step that begins tile it (its buffer held tile it-1, read to the end by
  // then), and is waited for before the barrier ending tile it+1's first step.
  const float c_scale = a.scale_log2;
  // need: the tile takes the mask.  That includes every tile dead for the
  // wave's keys (causal: all its queries before the first of those keys; or
  // those keys all at or past valid_len): it runs fully masked, so its
  // weights are exact zeros and the loop needs no branch around matrix work.
  auto tile = [&](const ItCur& c, bool& need, int& rel_h) {
    const int ti = c.ti;
    const long long qp0 = qpos(a, ti * kTile);
    need = kw_hi >= a.valid_len || (a.causal && kw_hi > qp0);
    int rel = 0;
    if (kpos >= a.valid_len) rel = kTile;
    else if (a.causal) rel = (int)max(0LL, min((long long)kTile, kpos - qp0));
    rel_h = rel - 4 * half;
  };
  // vector-memory operations of one tile copy issued by this wave
  auto wait_copy = [&](bool newer) {
    if (!newer) wait_vmcnt<0>();
    else if (wave < 2) wait_vmcnt<2 * PC::DMA + 1>();
    else wait_vmcnt<2 * PC::DMA>();
  };
  ItCur cq = it_start(hk * G), ct = cq;  // the next copy's iteration, tile()'s
  if (n_it > 0) copy_q(cq, base);
  it_next(cq);
  if (n_it > 1) copy_q(cq, base + PC::BUF);
  it_next(cq);
  wait_copy(n_it > 1);
  pipeline_barrier();  // tile 0 is in LDS
  // role 0: P of halves 0 and 1; role 1: dP and D of the half whose dS is
  // formed next (A: half 0, B: half 1)
  bf16x8 p0[2], p1[2];
  f32x16 scA = f32x16{}, scB = f32x16{};
  u32x4 stA[4] = {}, stB[4] = {};
  bool need = false;
  int rel_h = 0;
  if (n_it > 0) tile(ct, need, rel_h);
  pair_step<D, ROLE, 0, 1>(w, n_it > 0, false, 0, 0, need, rel_h, c_scale, p0, p1, scA, stA, scB,
                           stB);
  pipeline_barrier();  // P of tile 0, half 0
  unsigned bo = 0;     // buffer of tile it
  // Every tile but the last: both parts of both steps always run (dead
  // tiles fully masked, as above).
  for (int it = 0; it + 1 < n_it; ++it) {
    const unsigned bo_n = bo + PC::BUF == PC::NBUF * PC::BUF ? 0 : bo + PC::BUF;
    if (it + 2 < n_it) {
      copy_q(cq, base + (bo_n + PC::BUF == PC::NBUF * PC::BUF ? 0 : bo_n + PC::BUF));
      it_next(cq);
    }
    // step 1: half 1 of tile it forward, half 0 backward
    step_both<D, ROLE, 1, 0>(w, bo, bo, need, rel_h, c_scale, p1, p0, scB, stB, scA, stA);
    wait_copy(it + 2 < n_it);
    pipeline_barrier();  // P of half 1; tile it+1 is in LDS
    // step 2: half 0 of tile it+1 forward, half 1 of tile it backward
    it_next(ct);
    tile(ct, need, rel_h);
    step_both<D, ROLE, 0, 1>(w, bo_n, bo, need, rel_h, c_scale, p0, p1, scA, stA, scB, stB);
    pipeline_barrier();  // P of tile it+1, half 0; tile it read to the end
    bo = bo_n;
  }
  if (n_it > 0) {
    // the last tile: its second half, then nothing new
    step_both<D, ROLE, 1, 0>(w, bo, bo, need, rel_h, c_scale, p1, p0, scB, stB, scA, stA);
    pipeline_barrier();  // P of half 1
    pair_step<D, ROLE, 0, 1>(w, false, true, bo, bo, need, rel_h, c_scale, p0, p1, scA, stA, scB,
                             stB);
    pipeline_barrier();
  }

  if (key_ok) {
    const long long off = ((long long)b * a.kv_rows_b + kr) * HDkv + (long long)hk * D;
    float* dst = (ROLE == 1 ? kb.dk : kb.dv) + off;
    const float f = ROLE == 1 ? a.scale : 1.0f;
#pragma unroll
    for (int d = 0; d < C::NDT; ++d)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        float4* p = (float4*)(dst + 32 * d + 8 * gg + 4 * half);
        float4 x = *p;
        x.x += f * w.acc[d][4 * gg + 0];
        x.y += f * w.acc[d][4 * gg + 1];
        x.z += f * w.acc[d][4 * gg + 2];
        x.w += f * w.acc[d][4 * gg + 3];
        *p = x;
      }
  }
}

template <int D>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bwd_dkv_pair(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[PairCfg<D>::LDS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave < 4) pair_body<D, 0>(a, smem, wave, lane);
  else pair_body<D, 1>(a, smem, wave, lane);
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same gradients with no rounding of P or dS (the fp32
// tier of the checks).  Plain LDS-tiled vector arithmetic over 32 x 32
// (query, key) tiles, 8 threads per query or key row; not tuned for speed.
// Same launches as the bf16 path: the dq kernel also writes the row
// statistics, which the dk/dv kernel then reads.
// ---------------------------------------------------------------------------
constexpr int kF32T = 32;         // rows of a query or key tile
constexpr int kF32Threads = 256;  // 8 threads per row of a tile

template <int D>
struct F32Bwd {
  static constexpr int LD = D + 1;  // padded LDS row (floats): rows on distinct banks
  static constexpr int FPT = D / 8;  // features each thread owns (d = part + 8 m)
};

// Key row kr of block kb seen by a query at global position qp.
__device__ __forceinline__ bool f32_visible(const BwdArgs& a, const BwdBlock& kb, int kr,
                                            long long qp) {
  const long long kp = kb.k_pos0 + kr;
  return kr < kb.len && kp < a.valid_len && (!a.causal || kp <= qp);
}

// Rows row0 .. row0+31 of head h (zero past Sq) into t[32][LD].
template <int D>
__device__ __forceinline__ void f32_load_rows(float (*t)[F32Bwd<D>::LD], const float* base,
                                              long long row_stride, int rows_total, int row0,
                                              int tid) {
  for (int e = tid; e < kF32T * D; e += kF32Threads) {
    const int i = e / D, d = e % D, r = row0 + i;
    t[i][d] = r < rows_total ? base[(long long)r * row_stride + d] : 0.0f;
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void ring_attn_bwd_dq_f32(const BwdArgs a) {
  using C = F32Bwd<D>;
  __shared__ float sq[kF32T][C::LD], sdo[kF32T][C::LD], sk[kF32T][C::LD], sv[kF32T][C::LD];
  __shared__ float sds[kF32T][kF32T + 1];
  __shared__ float slse[kF32T], sdsum[kF32T];
  __shared__ long long sqp[kF32T];
  const int tid = threadIdx.x;
  const int n_qt = (a.Sq + kF32T - 1) / kF32T;
  const int qt = blockIdx.x % n_qt, bh = blockIdx.x / n_qt;
  const int b = bh / a.H, h = bh % a.H, hk = h / (a.H / a.Hkv);
  const int row0 = qt * kF32T;
  const long long HD = (long long)a.H * D, HDkv = (long long)a.Hkv * D;
  const float* q = (const float*)a.q + (long long)b * a.Sq * HD + (long long)h * D;
  const float* dout = (const float*)a.dout + (long long)b * a.Sq * HD + (long long)h * D;
  const float* o = (const float*)a.o + (long long)b * a.Sq * HD + (long long)h * D;
  f32_load_rows<D>(sq, q, HD, a.Sq, row0, tid);
  f32_load_rows<D>(sdo, dout, HD, a.Sq, row0, tid);
  const int ti = tid >> 3, part = tid & 7;  // this thread's query row and part
  {
    // row statistics, as the bf16 kernel forms them: base-2 lse (+inf for
    // a row that saw no key and for a padding query) and D = rowsum(dO O)
    // (0 for a padding query)
    const int r = row0 + ti;
    float dsum = 0.0f;
    if (r < a.Sq)
      for (int d = part; d < D; d += 8) dsum += dout[(long long)r * HD + d] * o[(long long)r * HD + d];
    dsum += __shfl_xor(dsum, 1);
    dsum += __shfl_xor(dsum, 2);
    dsum += __shfl_xor(dsum, 4);
    if (part == 0) {
      float lse2 = INFINITY;
      long long qp = LLONG_MAX;
      if (r < a.Sq) {
        qp = qpos(a, r);
        const bool real = qp < a.valid_len;
        const float l = a.lse[((long long)b * a.Sq + r) * a.H + h];
        lse2 = l == -INFINITY || !real ? INFINITY : l * kLog2e;
        if (!real) dsum = 0.0f;
        const long long so = ((long long)b * a.H + h) * a.Sq + r;
        a.stats[so] = lse2;
        a.stats[(long long)a.B * a.H * a.Sq + so] = -dsum;
      }
      slse[ti] = lse2;
      sdsum[ti] = dsum;
      sqp[ti] = qp;
    }
  }
  const long long q_hi = qpos(a, min(row0 + kF32T, a.Sq) - 1);
  float acc[C::FPT];
#pragma unroll
  for (int m = 0; m < C::FPT; ++m) acc[m] = 0.0f;
  for (int bi = 0; bi < a.nblk; ++bi) {
    const BwdBlock& kb = a.blk[bi];
    const float* kp = (const float*)kb.k + (long long)b * a.kv_rows_b * HDkv + (long long)hk * D;
    const float* vp = (const float*)kb.v + (long long)b * a.kv_rows_b * HDkv + (long long)hk * D;
    for (int k0 = 0; k0 < kb.len; k0 += kF32T) {
      // tiles wholly in the future of the tile's last query, or wholly
      // padding, hold no visible key (and neither do the later ones)
      if ((a.causal && kb.k_pos0 + k0 > q_hi) || kb.k_pos0 + k0 >= a.valid_len) break;
      __syncthreads();  // the previous tile's readers are done
      f32_load_rows<D>(sk, kp, HDkv, kb.len, k0, tid);
      f32_load_rows<D>(sv, vp, HDkv, kb.len, k0, tid);
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = part + 8 * e;
        float sc = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          sc += sq[ti][d] * sk[j][d];
          dp += sdo[ti][d] * sv[j][d];
        }
        float ds = 0.0f;
        if (f32_visible(a, kb, k0 + j, sqp[ti])) {
          const float pr = exp2f(sc * a.scale_log2 - slse[ti]);
          ds = pr * (dp - sdsum[ti]);
        }
        sds[ti][j] = ds;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < C::FPT; ++m) {
        const int d = part + 8 * m;
        float x = 0.0f;
        for (int j = 0; j < kF32T; ++j) x += sds[ti][j] * sk[j][d];
        acc[m] += x;
      }
    }
  }
  const int r = row0 + ti;
  if (r < a.Sq) {
    float* dq = a.dq + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int m = 0; m < C::FPT; ++m) dq[part + 8 * m] += a.scale * acc[m];
  }
}

// One workgroup per (visited block, batch, K/V head, 32 keys): walks every
// query tile of every query head of the group (those wholly before its keys
// skipped when causal) and accumulates dK and dV of its keys.
template <int D>
__global__ __launch_bounds__(kF32Threads) void ring_attn_bwd_dkv_f32(const BwdArgs a) {
  using C = F32Bwd<D>;
  __shared__ float sk[kF32T][C::LD], sv[kF32T][C::LD], sq[kF32T][C::LD], sdo[kF32T][C::LD];
  __shared__ float sp[kF32T][kF32T + 1], sds[kF32T][kF32T + 1];
  __shared__ float slse[kF32T], sdsum[kF32T];
  __shared__ long long sqp[kF32T];
  const int tid = threadIdx.x;
  int id = blockIdx.x;
  const int kt = id % a.n_ktiles;
  id /= a.n_ktiles;
  const int bi = id % a.nblk;
  id /= a.nblk;
  const int hk = id % a.Hkv, b = id / a.Hkv;
  const int G = a.H / a.Hkv;
  const BwdBlock& kb = a.blk[bi];
  const int k0 = kt * kF32T;
  if (k0 >= kb.len) return;  // a shorter block (uniform)
  const long long HD = (long long)a.H * D, HDkv = (long long)a.Hkv * D;
  const long long kvoff = (long long)b * a.kv_rows_b * HDkv + (long long)hk * D;
  f32_load_rows<D>(sk, (const float*)kb.k + kvoff, HDkv, kb.len, k0, tid);
  f32_load_rows<D>(sv, (const float*)kb.v + kvoff, HDkv, kb.len, k0, tid);
  const int tj = tid >> 3, part = tid & 7;  // this thread's key row and part
  const long long k_lo = kb.k_pos0 + k0;
  float dk[C::FPT], dv[C::FPT];
#pragma unroll
  for (int m = 0; m < C::FPT; ++m) dk[m] = dv[m] = 0.0f;
  const int n_qt = (a.Sq + kF32T - 1) / kF32T;
  const long long nst = (long long)a.B * a.H * a.Sq;
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const float* q = (const float*)a.q + (long long)b * a.Sq * HD + (long long)h * D;
    const float* dout = (const float*)a.dout + (long long)b * a.Sq * HD + (long long)h * D;
    for (int qt = 0; qt < n_qt; ++qt) {
      const int row0 = qt * kF32T;
      if (a.causal && qpos(a, min(row0 + kF32T, a.Sq) - 1) < k_lo) continue;
      __syncthreads();  // the previous tile's readers are done
      f32_load_rows<D>(sq, q, HD, a.Sq, row0, tid);
      f32_load_rows<D>(sdo, dout, HD, a.Sq, row0, tid);
      if (tid < kF32T) {
        const int r = row0 + tid;
        const long long so = ((long long)b * a.H + h) * a.Sq + r;
        slse[tid] = r < a.Sq ? a.stats[so] : INFINITY;
        sdsum[tid] = r < a.Sq ? -a.stats[nst + so] : 0.0f;
        sqp[tid] = r < a.Sq ? qpos(a, r) : LLONG_MAX;
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = part + 8 * e;
        float sc = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          sc += sk[tj][d] * sq[i][d];
          dp += sv[tj][d] * sdo[i][d];
        }
        float pr = 0.0f, ds = 0.0f;
        if (f32_visible(a, kb, k0 + tj, sqp[i])) {
          pr = exp2f(sc * a.scale_log2 - slse[i]);
          ds = pr * (dp - sdsum[i]);
        }
        sp[tj][i] = pr;
        sds[tj][i] = ds;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < C::FPT; ++m) {
        const int d = part + 8 * m;
        float xv = 0.0f, xk = 0.0f;
        for (int i = 0; i < kF32T; ++i) {
          xv += sp[tj][i] * sdo[i][d];
          xk += sds[tj][i] * sq[i][d];
        }
        dv[m] += xv;
        dk[m] += xk;
      }
    }
  }
  const int kr = k0 + tj;
  if (kr < kb.len) {
    const long long off = ((long long)b * a.kv_rows_b + kr) * HDkv + (long long)hk * D;
#pragma unroll
    for (int m = 0; m < C::FPT; ++m) {
      kb.dk[off + part + 8 * m] += a.scale * dk[m];
      kb.dv[off + part + 8 * m] += dv[m];
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Checks shared by both entry points (errors before any launch).
ra_status check_common(const char* name, int B, int Sq, int H, int D, ra_dtype dt) {
  if (B < 0 || Sq < 0 || H < 0)
    return ra::fail(RA_ERR_SHAPE, "%s: negative size (B=%d Sq=%d H=%d)", name, B, Sq, H);
  if (dt != RA_BF16 && dt != RA_FP32) return ra::fail(RA_ERR_DTYPE, "%s: unknown dtype %d", name, (int)dt);
  if (D != 64 && D != 128)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: head dimension %d not supported (64 or 128)", name, D);
  return RA_OK;
}

void set_scale(BwdArgs& a, float scale, int D) {
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale = (float)sc;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
}

// The three launches over a.nblk visited blocks of block_len rows each.
ra_status launch_bwd(const char* name, BwdArgs& a, int D, ra_dtype dt, int block_len,
                     hipStream_t s) {
  if (dt == RA_FP32) {
    const long long n_dq = (long long)a.B * a.H * ((a.Sq + kF32T - 1) / kF32T);
    a.n_ktiles = (block_len + kF32T - 1) / kF32T;
    const long long n_dkv = (long long)a.nblk * a.B * a.Hkv * a.n_ktiles;
    if (n_dq > 0x7fffffffLL || n_dkv > 0x7fffffffLL)
      return ra::fail(RA_ERR_UNSUPPORTED, "%s: grid too large", name);
    const dim3 gq((unsigned)n_dq), gk((unsigned)n_dkv);
    if (D == 128) hipLaunchKernelGGL(ring_attn_bwd_dq_f32<128>, gq, dim3(kF32Threads), 0, s, a);
    else hipLaunchKernelGGL(ring_attn_bwd_dq_f32<64>, gq, dim3(kF32Threads), 0, s, a);
    if (n_dkv > 0) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bwd_dkv_f32<128>, gk, dim3(kF32Threads), 0, s, a);
      else hipLaunchKernelGGL(ring_attn_bwd_dkv_f32<64>, gk, dim3(kF32Threads), 0, s, a);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
      return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    return RA_OK;
  }
  // RA_OPT_ATTN_WAVES (4 or 8) forces the dQ workgroup size as it does the
  // forward's
  const int forced = ra::option(RA_OPT_ATTN_WAVES);
  const bool dq8 = forced ? forced == 8 : (long long)a.B * a.H * ((a.Sq + 255) / 256) >= 256;
  const long long n_dq = (long long)a.B * a.H * ((a.Sq + (dq8 ? 255 : 127)) / (dq8 ? 256 : 128));
  a.n_ktiles = (block_len + kRows - 1) / kRows;
  const long long n_dkv = (long long)a.nblk * a.B * a.Hkv * a.n_ktiles;
  if (n_dq > 0x7fffffffLL || n_dkv > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: grid too large", name);
  if (a.lockstep == 0) {  // not preset by the caller (the zigzag share)
    a.lockstep = 1;
    for (int i = 1; i < a.nblk; ++i) {
      const long long k_end = a.blk[i].k_pos0 + a.blk[i].len;  // one past its last key
      if ((a.causal && k_end - 1 > a.q_pos0) || k_end > a.valid_len) a.lockstep = 0;
    }
  }
  // dq first: it writes the row statistics that the dk/dv kernels read
  const dim3 gq((unsigned)n_dq);
  if (dq8) {
    if (D == 128) hipLaunchKernelGGL((ring_attn_bwd_dq<128, 8>), gq, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((ring_attn_bwd_dq<64, 8>), gq, dim3(512), 0, s, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((ring_attn_bwd_dq<128, 4>), gq, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ring_attn_bwd_dq<64, 4>), gq, dim3(256), 0, s, a);
  }
  if (n_dkv > 0) {
    const dim3 g((unsigned)n_dkv);
    if (D == 128) hipLaunchKernelGGL(ring_attn_bwd_dkv_pair<128>, g, dim3(kPairThreads), 0, s, a);
    else hipLaunchKernelGGL(ring_attn_bwd_dkv_pair<64>, g, dim3(kPairThreads), 0, s, a);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
  return RA_OK;
}

}  // namespace

extern "C" ra_status ra_block_attn_bwd(const void* q, const void* k, const void* v,
                                       const void* o, const void* dout, const float* lse,
                                       int B, int Sq, int Sk, int H, int D, ra_dtype dt,
                                       float scale, long long q_pos0, long long k_pos0,
                                       int causal, long long valid_len, float* dq, float* dk,
                                       float* dv, float* stats_ws, void* stream) {
  static const char* name = "ra_block_attn_bwd";
  ra::clear_error();
  ra_status st = check_common(name, B, Sq, H, D, dt);
  if (st != RA_OK) return st;
  if (Sk < 0) return ra::fail(RA_ERR_SHAPE, "%s: negative size (Sk=%d)", name, Sk);
  if ((long long)B * Sq * H == 0 || Sk == 0) return RA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !stats_ws)
    return ra::fail(RA_ERR_NULL, "%s: NULL argument", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ra::fail(RA_ERR_SHAPE, "%s: tensors must be 16-byte aligned", name);
  if (valid_len < 0) valid_len = LLONG_MAX;
  BwdArgs a{};
  a.q = q;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.stats = stats_ws;
  a.q_pos0 = q_pos0;
  a.q_pos1 = q_pos0 + Sq;
  a.q_split = Sq;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
  a.Hkv = H;
  a.kv_rows_b = Sk;
  a.causal = causal != 0;
  set_scale(a, scale, D);
  // a block with no visible pair ([RA] §3.4 SKIP) is neither read nor written
  a.nblk = 0;
  if (ra::block_class(q_pos0, q_pos0 + Sq, k_pos0, k_pos0 + Sk, causal != 0, valid_len) != RA_SKIP)
    a.blk[a.nblk++] = BwdBlock{k, v, dk, dv, k_pos0, Sk, 0};
  if (a.nblk == 0) return RA_OK;
  return launch_bwd(name, a, D, dt, Sk, (hipStream_t)stream);
}

namespace {
// The ring backward of one rank (shared by the MHA and GQA entry points).
ra_status ring_bwd(const char* name, const void* q_r, const void* const* k_blocks,
                   const void* const* v_blocks, const void* o_r, const void* do_r,
                   const float* lse_r, int B, int Sb, int H, int Hkv, int D, int P, int rank,
                   ra_dtype dt, float scale, int causal, long long valid_len, float* dq_r,
                   float* const* dk_blocks, float* const* dv_blocks, float* stats_ws,
                   void* stream) {
  ra::clear_error();
  ra_status st = check_common(name, B, Sb, H, D, dt);
  if (st != RA_OK) return st;
  if (Hkv <= 0 || H % Hkv != 0)
    return ra::fail(RA_ERR_SHAPE, "%s: %d query heads are not a multiple of %d K/V heads",
                    name, H, Hkv);
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (P > RA_MAX_P) return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P=%d", name, P, RA_MAX_P);
  if (rank < 0 || rank >= P) return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  if ((long long)B * Sb * H == 0) return RA_OK;
  if (!q_r || !o_r || !do_r || !lse_r || !dq_r || !stats_ws || !k_blocks || !v_blocks ||
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
  a.stats = stats_ws;
  a.q_pos0 = (long long)rank * Sb;
  a.q_pos1 = a.q_pos0 + Sb;
  a.q_split = Sb;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sb;
  a.H = H;
  a.Hkv = Hkv;
  a.kv_rows_b = Sb;
  a.causal = causal != 0;
  set_scale(a, scale, D);
  // the ring schedule of [RA] §3.3 with the classes of §3.4; SKIP blocks
  // are neither read nor written
  int src[RA_MAX_P], cls[RA_MAX_P];
  st = ra_ring_schedule(P, rank, Sb, causal, valid_len, src, cls);
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
  return launch_bwd(name, a, D, dt, Sb, (hipStream_t)stream);
}
}  // namespace

extern "C" ra_status ra_ring_attn_bwd(const void* q_r, const void* const* k_blocks,
                                      const void* const* v_blocks, const void* o_r,
                                      const void* do_r, const float* lse_r, int B, int Sb,
                                      int H, int D, int P, int rank, ra_dtype dt, float scale,
                                      int causal, long long valid_len, float* dq_r,
                                      float* const* dk_blocks, float* const* dv_blocks,
                                      float* stats_ws, void* stream) {
  return ring_bwd("ra_ring_attn_bwd", q_r, k_blocks, v_blocks, o_r, do_r, lse_r, B, Sb, H, H, D,
                  P, rank, dt, scale, causal, valid_len, dq_r, dk_blocks, dv_blocks, stats_ws,
                  stream);
}

extern "C" ra_status ra_ring_attn_bwd_gqa(const void* q_r, const void* const* k_blocks,
                                          const void* const* v_blocks, const void* o_r,
                                          const void* do_r, const float* lse_r, int B, int Sb,
                                          int H, int H_kv, int D, int P, int rank, ra_dtype dt,
                                          float scale, int causal, long long valid_len,
                                          float* dq_r, float* const* dk_blocks,
                                          float* const* dv_blocks, float* stats_ws,
                                          void* stream) {
  return ring_bwd("ra_ring_attn_bwd_gqa", q_r, k_blocks, v_blocks, o_r, do_r, lse_r, B, Sb, H,
                  H_kv, D, P, rank, dt, scale, causal, valid_len, dq_r, dk_blocks, dv_blocks,
                  stats_ws, stream);
}

extern "C" ra_status ra_zigzag_attn_bwd(const void* q_r, const void* const* k_shares,
                                        const void* const* v_shares, const void* o_r,
                                        const void* do_r, const float* lse_r, int B, int Sr,
                                        int H, int D, int P, int rank, ra_dtype dt, float scale,
                                        int causal, long long valid_len, float* dq_r,
                                        float* const* dk_shares, float* const* dv_shares,
                                        float* stats_ws, void* stream) {
  static const char* name = "ra_zigzag_attn_bwd";
  ra::clear_error();
  ra_status st = check_common(name, B, Sr, H, D, dt);
  if (st != RA_OK) return st;
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (2 * P > RA_MAX_P)
    return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P/2=%d", name, P, RA_MAX_P / 2);
  if (rank < 0 || rank >= P) return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  if (Sr % 128 != 0)
    return ra::fail(RA_ERR_SHAPE, "%s: rows per rank (%d) must be two chunks of a multiple "
                    "of 64 rows; pad the sequence to ra_zigzag_padded_len(S, P)", name, Sr);
  if ((long long)B * Sr * H == 0) return RA_OK;
  if (!q_r || !o_r || !do_r || !lse_r || !dq_r || !stats_ws || !k_shares || !v_shares ||
      !dk_shares || !dv_shares)
    return ra::fail(RA_ERR_NULL, "%s: NULL argument", name);
  if (!aligned16(q_r) || !aligned16(o_r) || !aligned16(do_r) || !aligned16(dq_r))
    return ra::fail(RA_ERR_SHAPE, "%s: q, o, do and dq must be 16-byte aligned", name);
  const int c = Sr / 2;  // chunk length
  const long long S = (long long)P * Sr;
  if (valid_len < 0 || valid_len > S) valid_len = S;
  BwdArgs a{};
  a.q = q_r;
  a.o = o_r;
  a.dout = do_r;
  a.lse = lse_r;
  a.dq = dq_r;
  a.stats = stats_ws;
  // the share is chunk rank (rows [0, c)) then chunk 2P-1-rank (rows [c, 2c))
  a.q_pos0 = (long long)rank * c;
  a.q_pos1 = (long long)(2 * P - 1 - rank) * c;
  a.q_split = c;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sr;
  a.H = H;
  a.Hkv = H;
  a.kv_rows_b = Sr;
  a.causal = causal != 0;
  set_scale(a, scale, D);
  // the zigzag ring: round t visits the share of rank (rank - t) mod P, each
  // share two chunks classified against the whole query share; the dK/dV
  // parts of a chunk go to the matching rows of its share's buffers
  int src[RA_MAX_P], cls[2 * RA_MAX_P];
  st = ra_zigzag_schedule(P, rank, c, causal, valid_len, src, cls);
  if (st != RA_OK) return st;
  a.nblk = 0;
  const size_t in_row = (size_t)H * D * (dt == RA_FP32 ? 4 : 2), g_row = (size_t)H * D;
  for (int t = 0; t < P; ++t) {
    const int j = src[t];
    for (int half = 0; half < 2; ++half) {
      if (cls[2 * t + half] == RA_SKIP) continue;
      if (!k_shares[j] || !v_shares[j] || !dk_shares[j] || !dv_shares[j])
        return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited share %d", name, j);
      if (!aligned16(k_shares[j]) || !aligned16(v_shares[j]) || !aligned16(dk_shares[j]) ||
          !aligned16(dv_shares[j]))
        return ra::fail(RA_ERR_SHAPE, "%s: share %d not 16-byte aligned", name, j);
      const int chunk = half == 0 ? j : 2 * P - 1 - j;
      const size_t r0 = (size_t)half * c;
      a.blk[a.nblk++] = BwdBlock{(const char*)k_shares[j] + r0 * in_row,
                                 (const char*)v_shares[j] + r0 * in_row, dk_shares[j] + r0 * g_row,
                                 dv_shares[j] + r0 * g_row, (long long)chunk * c, c, 0};
    }
  }
  // causal: the table starts with the share's own two chunks, so the later
  // query tiles of the lockstep order start from the third entry
  if (causal && a.nblk >= 2 && cls[0] != RA_SKIP && cls[1] != RA_SKIP) a.lockstep = 2;
  return launch_bwd(name, a, D, dt, c, (hipStream_t)stream);
}

extern "C" ra_status ra_ring_attn_bwd_varlen(const void* q_r, const void* const* k_blocks,
                                             const void* const* v_blocks, const void* o_r,
                                             const void* do_r, const float* lse_r, int Sb, int H,
                                             int D, int P, int rank, ra_dtype dt, float scale,
                                             int causal, const long long* cu_seqlens,
                                             int n_seqs, float* dq_r, float* const* dk_blocks,
                                             float* const* dv_blocks, float* stats_ws,
                                             void* stream) {
  static const char* name = "ra_ring_attn_bwd_varlen";
  ra::clear_error();
  ra_status st = check_common(name, 1, Sb, H, D, dt);
  if (st != RA_OK) return st;
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (P > RA_MAX_P) return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P=%d", name, P, RA_MAX_P);
  if (rank < 0 || rank >= P) return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  if (n_seqs < 0 || (n_seqs > 0 && !cu_seqlens))
    return ra::fail(RA_ERR_NULL, "%s: NULL or negative sample table", name);
  const long long S = (long long)P * Sb;
  for (int i = 0; i < n_seqs; ++i)
    if (cu_seqlens[i] > cu_seqlens[i + 1] || cu_seqlens[i] < 0)
      return ra::fail(RA_ERR_SHAPE, "%s: sample boundaries must increase from 0", name);
  if (n_seqs > 0 && (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] > S))
    return ra::fail(RA_ERR_SHAPE, "%s: samples must start at 0 and end within P*Sb = %lld",
                    name, S);
  if ((long long)Sb * H == 0) return RA_OK;
  if (!q_r || !o_r || !do_r || !lse_r || !dq_r || !stats_ws || !k_blocks || !v_blocks ||
      !dk_blocks || !dv_blocks)
    return ra::fail(RA_ERR_NULL, "%s: NULL argument", name);
  if (!aligned16(q_r) || !aligned16(o_r) || !aligned16(do_r) || !aligned16(dq_r))
    return ra::fail(RA_ERR_SHAPE, "%s: q, o, do and dq must be 16-byte aligned", name);
  const long long q0 = (long long)rank * Sb, q1 = q0 + Sb;
  int src[RA_MAX_P], cls[RA_MAX_P];
  st = ra_ring_schedule(P, rank, Sb, causal, S, src, cls);
  if (st != RA_OK) return st;
  const size_t in_row = (size_t)H * D * (dt == RA_FP32 ? 4 : 2), g_row = (size_t)H * D;
  // one launch pair per sample that meets the rank's rows: its rows of the
  // share against the parts of the visited blocks inside that sample, in
  // ring order (the forward's split, so each sample's gradients use only
  // its own pairs)
  for (int i = 0; i < n_seqs; ++i) {
    const long long s0 = cu_seqlens[i], s1 = cu_seqlens[i + 1];
    const long long r0 = s0 > q0 ? s0 : q0, r1 = s1 < q1 ? s1 : q1;
    if (r1 <= r0) continue;
    BwdArgs a{};
    a.q = (const char*)q_r + (size_t)(r0 - q0) * in_row;
    a.o = (const char*)o_r + (size_t)(r0 - q0) * in_row;
    a.dout = (const char*)do_r + (size_t)(r0 - q0) * in_row;
    a.lse = lse_r + (r0 - q0) * H;
    a.dq = dq_r + (r0 - q0) * g_row;
    a.stats = stats_ws;
    a.q_pos0 = r0;
    a.q_pos1 = r1;
    a.q_split = (int)(r1 - r0);
    a.valid_len = s1;  // keys past the sample's end are not real for it
    a.B = 1;
    a.Sq = (int)(r1 - r0);
    a.H = H;
    a.Hkv = H;
    a.kv_rows_b = Sb;  // B = 1: never used for a stride
    a.causal = causal != 0;
    set_scale(a, scale, D);
    a.nblk = 0;
    int max_len = 0;
    for (int t = 0; t < P; ++t) {
      if (cls[t] == RA_SKIP) continue;
      const int j = src[t];
      const long long b0 = (long long)j * Sb, b1 = b0 + Sb;
      const long long k0 = b0 > s0 ? b0 : s0, k1 = b1 < s1 ? b1 : s1;
      if (k1 <= k0) continue;
      if (ra::block_class(r0, r1, k0, k1, causal != 0, s1) == RA_SKIP) continue;
      if (!k_blocks[j] || !v_blocks[j] || !dk_blocks[j] || !dv_blocks[j])
        return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited block %d", name, j);
      if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]) || !aligned16(dk_blocks[j]) ||
          !aligned16(dv_blocks[j]))
        return ra::fail(RA_ERR_SHAPE, "%s: block %d not 16-byte aligned", name, j);
      const size_t off = (size_t)(k0 - b0);
      a.blk[a.nblk++] = BwdBlock{(const char*)k_blocks[j] + off * in_row,
                                 (const char*)v_blocks[j] + off * in_row,
                                 dk_blocks[j] + off * g_row, dv_blocks[j] + off * g_row, k0,
                                 (int)(k1 - k0), 0};
      if (k1 - k0 > max_len) max_len = (int)(k1 - k0);
    }
    if (a.nblk == 0) continue;
    st = launch_bwd(name, a, D, dt, max_len, (hipStream_t)stream);
    if (st != RA_OK) return st;
  }
  return RA_OK;
}
