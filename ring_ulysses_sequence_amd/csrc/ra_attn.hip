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

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

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
  // global position of query row r: q_pos0 + r for r < q_split, else
  // q_pos1 + (r - q_split) (two segments for the zigzag share; q_split is a
  // multiple of 64 and q_pos1 >= q_pos0 + q_split, so positions increase
  // with the row)
  long long q_pos0;
  long long q_pos1;
  int q_split;
  int kv_rows_b;       // rows between consecutive batches in every K/V buffer
  int Hkv;             // K/V heads (H % Hkv == 0): query head h reads K/V head
                       // h / (H / Hkv)
  long long valid_len; // keys at global positions >= valid_len are padding
  int B, Sq, H;
  int n_qtiles;
  int causal;
  int o_fp32;
  float scale_log2;    // scale * log2(e): scores live in the base-2 domain
  // split ring (nsplit > 1): the visited-tile sequence of every 128-row
  // query tile is cut into nsplit near-equal runs, one workgroup each; run
  // j of query tile qt of (b, h) writes its fp32 partial (o normalised, lse)
  // to slot ((b*H + h)*n_qtiles + qt)*nsplit + j of o / lse ([slot][128
  // rows][D] and [slot][128 rows]).
  int nsplit;
  int nblk;
  KVBlock blk[RA_MAX_P];
};

constexpr float kLn2 = 0.693147180559945309f;

__host__ __device__ __forceinline__ long long qpos(const AttnArgs& a, int row) {
  return row < a.q_split ? a.q_pos0 + row : a.q_pos1 + (row - a.q_split);
}

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
__host__ __device__ __forceinline__ int tiles_of(const AttnArgs& a, int b, long long q_hi) {
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
// of work, so the workgroups resident on one XCD share K/V in that XCD's L2.
// Within the range, work goes in groups of kHeadGroup heads: the group's
// query tiles are taken kTileRun at a time from each of its heads in turn,
// later tiles (more causal work) first.  The workgroups resident together
// then cover a few heads with neighbouring query tiles, which walk the same
// K/V tiles at nearly the same time (measured: ~4 % over whole heads in
// turn on the long-context share).  Shapes that do not divide evenly take
// the heads one after another.
constexpr int kHeadGroup = 4, kTileRun = 8;

__device__ __forceinline__ void tile_coords(const AttnArgs& a, int id, int n, int& b, int& h,
                                            int& qt) {
  if ((n & 7) == 0) id = (id & 7) * (n >> 3) + (id >> 3);
  const int Q = a.n_qtiles, BH = a.B * a.H;
  int bh;
  if (Q % kTileRun == 0 && BH % kHeadGroup == 0) {
    const int g = id / (kHeadGroup * Q), r = id % (kHeadGroup * Q);
    const int run = r / (kHeadGroup * kTileRun);
    bh = g * kHeadGroup + (r / kTileRun) % kHeadGroup;
    qt = Q - 1 - (run * kTileRun + r % kTileRun);
  } else {
    bh = id / Q;
    qt = Q - 1 - id % Q;
  }
  h = bh % a.H;
  b = bh / a.H;
}
__device__ __forceinline__ void tile_coords(const AttnArgs& a, int& b, int& h, int& qt) {
  tile_coords(a, (int)blockIdx.x, (int)gridDim.x, b, h, qt);
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
// K and V tiles (64 keys x D, row-major as in HBM) are copied HBM -> LDS by
// the buffer unit itself (buffer_load ... lds: each lane's 16 bytes land at
// LDS base + 16*lane), so staging costs no registers and no VALU work, and
// rows past the end of a block come back as zeros from the buffer range
// check.  The copy picks, for every LDS position, the global 16-byte chunk
// that belongs there under an XOR swizzle that keeps the matrix-core operand
// reads free of bank conflicts:
//   K: chunk c of key row r is stored at chunk c ^ (r & 15)          (D = 128)
//                                          c ^ ((r >> 1) & 7)        (D = 64)
//   V: chunk c of key row r is stored at chunk c ^ ((r & 3) << 2)    (D = 128)
//                                          c ^ (((r >> 1) & 1) << 2) (D = 64)
// K feeds S^T = K Q^T as the A operand with ds_read_b128.  V feeds
// O^T += V^T P^T as the A operand through ds_read_b64_tr_b16: inside each
// 16-lane group, lane j receives element j%4 of the 64-bit rows supplied by
// lanes j/4, j/4+4, j/4+8, j/4+12; supplier r = 4e + q points at
// V[key_e][d0 + 4q .. d0 + 4q + 3], so lane j gets V[key_0..3][d0 + j].
//
// Software pipeline (per wave, iteration n over the visited tiles):
//   LDS holds K(n+1), V(n) and V(n+1) (copied during iterations n-2, n-1);
//   copy K(n+2) and V(n+2) into the buffers freed by iteration n-1;
//   mask / row max / rescale of tile n's scores (already in registers);
//   S^T(n+1) = K(n+1) Q^T on the matrix cores, interleaved instruction by
//   instruction with the exponentials of tile n on the vector ALUs;
//   O^T += V(n)^T P(n)^T;
//   wait for this wave's K copy (the V copy may stay in flight), barrier.
// Two K buffers and three V buffers (80 KiB at D = 128, so two workgroups
// still share a CU).  Operand reads run four matrix ops ahead of their use.
// The loop is unrolled by two so the K parity and the score registers are
// constants; the V buffer index cycles mod 3 at run time.
template <int D, int NW>
struct Bf16Cfg {
  static constexpr int THREADS = 64 * NW;         // NW waves per workgroup
  static constexpr int BR = 32 * NW;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int ROWB = D * 2;              // bytes per key row in LDS
  static constexpr int TILE = BC * ROWB;          // one K or V tile
  static constexpr int KB = 0;                    // 2 K buffers at KB + p*TILE
  static constexpr int VB = 2 * TILE;             // 3 V buffers at VB + p*TILE
  static constexpr int LDS = 5 * TILE;
  static constexpr int CHUNKS = D / 8;            // 16-byte chunks per row
  static constexpr int DMA = TILE / 1024 / NW;     // 1 KiB copies per wave per tile
  static constexpr int NC = D / 16;               // k-steps of S^T = K Q^T
  static constexpr int NDT = D / 32;              // 32-row d tiles of O^T
  static constexpr int NS = BC / 2;               // scores per lane per tile
};

template <int D>
__device__ __forceinline__ int swz_k(int r, int c) {
  return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int swz_v(int r, int c) {
  return D == 128 ? (c ^ ((r & 3) << 2)) : (c ^ (((r >> 1) & 1) << 2));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access
constexpr float kRescaleSlack = 8.0f;   // lazy rescale threshold (base-2 units)

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ds_read_b64_tr_b16 as inline assembly.  The compiler's own form of this
// read makes it wait for every LDS-DMA copy in flight (it cannot tell which
// LDS bytes they write), which would stall each P V phase on the copies
// issued at the start of the same iteration.  Here the read is invisible to
// the compiler's wait insertion, so its result must be claimed with
// claim_lds<N> before use; the copies it must not overtake are ordered by
// the explicit waits and barriers of the pipeline.
__device__ __forceinline__ s16x4 lds_read_tr16(unsigned addr_lds) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr_lds));
  return r;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16(unsigned addr_lds) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr_lds), "n"(OFF));
  return r;
}
// Wait until at most N LDS (or scalar-memory) operations of this wave are
// outstanding, and make `x` depend on the wait so that no use of it is
// scheduled before.  LDS operations complete in issue order, so with N =
// the number of LDS reads issued after the one that produced x, x is ready.
template <int N, typename T>
__device__ __forceinline__ void claim_lds(T& x) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}
// Workgroup barrier for the copy pipeline.  The caller has already waited
// (vmcnt) for the copies that must be visible after it; unlike
// __syncthreads, this does not also wait for the copies that may stay in
// flight.  All of this wave's LDS reads have returned (lgkmcnt(0)), so the
// buffers they read may be overwritten once every wave has arrived.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Position in the visited-tile sequence: tile t (of n) of visited block blk.
struct Cursor {
  int blk, t, n;
};

// A workgroup's visited-tile sequence: the tiles of every visited block in
// ring order, each block up to the last tile with a key visible to the
// workgroup's last query q_hi.  The span ends before tile (end_blk, end_t):
// (a.nblk, 0) for the whole sequence.  A cursor past the span reads
// blk = a.nblk.
struct Span {
  long long q_hi;
  int end_blk, end_t;
};

// Position of tile number i of the sequence (blk = a.nblk past its end).
__device__ __forceinline__ Cursor seq_pos(const AttnArgs& a, long long q_hi, int i) {
  Cursor c{0, 0, 0};
  for (; c.blk < a.nblk; ++c.blk) {
    c.n = tiles_of<64>(a, c.blk, q_hi);
    if (i < c.n) break;
    i -= c.n;
  }
  c.t = i;
  return c;
}
__device__ __forceinline__ Cursor span_end(const AttnArgs& a, const Span& sp, Cursor c) {
  if (c.blk > sp.end_blk || (c.blk == sp.end_blk && c.t >= sp.end_t)) c.blk = a.nblk;
  return c;
}
__device__ __forceinline__ Cursor cursor_first(const AttnArgs& a, const Span& sp, int lo) {
  return span_end(a, sp, seq_pos(a, sp.q_hi, lo));
}
__device__ __forceinline__ Cursor cursor_next(const AttnArgs& a, const Span& sp, Cursor c) {
  if (c.blk >= a.nblk) return c;
  if (++c.t >= c.n) {
    c.t = 0;
    ++c.blk;
    while (c.blk < a.nblk && (c.n = tiles_of<64>(a, c.blk, sp.q_hi)) == 0) ++c.blk;
  }
  return span_end(a, sp, c);
}

// Everything a wave keeps in registers across tiles.
template <int D, int NW>
struct WaveState {
  using C = Bf16Cfg<D, NW>;
  bf16x8 qf[C::NC];        // Q fragment (B operand of S^T)
  f32x16 oacc[C::NDT];     // O^T accumulators (unnormalised u)
  float m_ref;             // reference max (base 2), -inf before any key
  float m_true;            // exact running max (base 2)
  float l_run;             // this lane's half of sum of bf16(2^(s - m_ref))
  int kaddr[C::NC];        // LDS byte offsets of the K operand reads
  int vaddr[C::NDT];       // LDS byte offsets of the V operand reads
  int voffk[C::DMA];       // copy source offsets (K) within a tile
  int voffv[C::DMA];       // copy source offsets (V) within a tile
};

// Copy one K or V tile (rows kt0 .. kt0+63 of batch b, head h of `src`, a
// visited block of `len` rows whose batches lie rows_b rows apart) into LDS
// at `dst`; each wave copies C::DMA KiB.
template <int D, int NW>
__device__ __forceinline__ void copy_tile(const void* src, int len, int rows_b, int ti, int b,
                                          int h, int H, int HD2, int wave, const int* voff,
                                          char* dst) {
  using C = Bf16Cfg<D, NW>;
  const int kt0 = ti * C::BC;
  const int rows = min(C::BC, len - kt0);
  const long long off = (((long long)b * rows_b + kt0) * H + h) * (D * 2);
  const int nrec = (rows - 1) * HD2 + D * 2;
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)src + off), 0, nrec, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < C::DMA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_ptr)(dst + (wave * C::DMA + i) * 1024), 16, voff[i], 0, 0, 0);
}

// S^T of one 64-key tile: the K tile at LDS byte offset kb times Q^T.
template <int D, int NW>
__device__ __forceinline__ void scores_tile(char* smem, int kb, const WaveState<D, NW>& w,
                                            f32x16 (&acc)[2]) {
  using C = Bf16Cfg<D, NW>;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    acc[kt] = f32x16{};
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const bf16x8 kf = *(const bf16x8*)(smem + kb + kt * 32 * C::ROWB + w.kaddr[c]);
      acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, w.qf[c], acc[kt], 0, 0, 0);
    }
  }
}

// Exponentials of one tile against the reference max, their bf16 copy P^T
// and the denominator over the same rounded weights ([RA] §3.2).
__device__ __forceinline__ void exp_tile(f32x16 (&s)[2], float m_use, float c_scale,
                                         bf16x8 (&pb)[4], float& l_run) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) s[kt][v] = fast_exp2(fmaf(s[kt][v], c_scale, -m_use));
#pragma unroll
  for (int G = 0; G < 4; ++G)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[G][e] = (__bf16)s[G >> 1][(G & 1) * 8 + e];
  float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
  for (int G = 0; G < 4; ++G)
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const bf16x2 p0 = {pb[G][e], pb[G][e + 1]}, p1 = {pb[G][e + 2], pb[G][e + 3]};
      l0 = __builtin_amdgcn_fdot2_f32_bf16(p0, kOnes2, l0, false);
      l1 = __builtin_amdgcn_fdot2_f32_bf16(p1, kOnes2, l1, false);
    }
  l_run += l0 + l1;
}

// Front half of pipeline step n: classification of tiles n and n+1, mask,
// row max and lazy rescale of tile n, then S^T(n+1) = K(n+1) Q^T on the
// matrix cores alongside the exponentials of tile n (P(n) into pb).  K(n+1)
// sits in K buffer PAR^1.  Returns whether tile n is live for this wave.
template <int D, int NW, int PAR>
__device__ __forceinline__ bool step_front(
    const AttnArgs& a, char* smem, WaveState<D, NW>& w, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
    const Cursor& t0, const Cursor& t1, long long wq_lo, long long wq_hi, int wrows, int col,
    int half, bf16x8 (&pb)[Bf16Cfg<D, NW>::NS / 8]) {
  using C = Bf16Cfg<D, NW>;
  constexpr int BC = C::BC;
  const float c_scale = a.scale_log2;
  // tile n: classification, mask, row max, lazy rescale
  const KVBlock& kb0 = a.blk[t0.blk];
  const int kt0 = t0.t * BC;
  const long long kp0 = kb0.k_pos0 + kt0;
  const bool live0 = wrows > 0 && !(a.causal && kp0 > wq_hi);
  bool live1 = false;
  if (t1.blk < a.nblk) {
    const long long kp1 = a.blk[t1.blk].k_pos0 + (long long)t1.t * BC;
    live1 = wrows > 0 && !(a.causal && kp1 > wq_hi);
  }
  float m_use = 0.0f;
  if (live0) {
    long long lim_ll = kb0.len - kt0;
    if (a.valid_len - kp0 < lim_ll) lim_ll = a.valid_len - kp0;
    if (lim_ll < BC || (a.causal && kp0 + BC - 1 > wq_lo)) {
      // key j of the tile is masked for this lane's query when
      // j > (query - first key) or j >= klim (32-bit, tile relative)
      const int klim = (int)max(0LL, lim_ll);
      int t = min(klim, BC) - 1 - 4 * half;
      if (a.causal) {
        // wave-uniform offset of the first query from the first key, clamped
        // on the scalar unit so the per-lane part stays 32-bit
        const long long d = wq_lo - kp0;
        const int dc = (int)(d < -2 * BC ? -2 * BC : (d > 2 * BC ? 2 * BC : d));
        const int rel = max(-1, dc + col - 4 * half);
        t = min(t, rel);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * kt + 8 * (v >> 2) + (v & 3) > t) s_cur[kt][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < C::NS; ++i) mx = fmaxf(mx, s_cur[i >> 4][i & 15]);
    mx = pair_max(mx) * c_scale;
    w.m_true = fmaxf(w.m_true, mx);
    const bool need = mx > w.m_ref + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // move the reference: u and l are rescaled together, so u / l keeps
      // the value of [RA] §3.2's recurrence while p = 2^(s - m_ref) <= 2^8
      // lanes that keep their reference use alpha = 1 (a lane still at
      // -inf must not form 2^(-inf - -inf))
      const float m_new = need ? mx : w.m_ref;
      const float alpha = need ? fast_exp2(w.m_ref - mx) : 1.0f;
      w.l_run *= alpha;
#pragma unroll
      for (int i = 0; i < C::NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) w.oacc[i][v] *= alpha;
      w.m_ref = m_new;
    }
    m_use = w.m_ref == -INFINITY ? 0.0f : w.m_ref;
  }
  // S^T(n+1) on the matrix cores alongside the exponentials of tile n
  constexpr int kbuf_next = C::KB + (PAR ^ 1) * C::TILE;
  if (live0 && live1) {
    // Explicit interleave: step i issues the K read of step i+2, the
    // matrix-core op of step i and 16/NC exponentials (with their bf16
    // conversion and denominator update); sched_barrier keeps the steps in
    // this order so the vector work of tile n fills the matrix-core
    // latency of tile n+1.
    constexpr int NSTEP = 2 * C::NC;
    constexpr int PER = C::NS / NSTEP;  // scores per step (2 for D=128)
    constexpr int PF = NSTEP >= 8 ? 4 : 2;  // operand read lead (matrix ops)
    bf16x8 kf[PF + 1];
    // step i works on score tile kt = i % 2 with k-step c = i / 2, so
    // consecutive matrix-core ops never depend on each other
    auto kread = [&](int i) -> bf16x8 {
      return *(const bf16x8*)(smem + kbuf_next + (i % 2) * 32 * C::ROWB + w.kaddr[i / 2]);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = kread(i);
    float lp[2] = {0.0f, 0.0f};
    float xs[3][PER];
#pragma unroll
    for (int t = 0; t < NSTEP + 2; ++t) {
      // slot t: matrix op t - 2 (slots 0, 1 run ahead of the first), shift of
      // group t, exponential of group t - 1, bf16 copy and sum of group t - 2
      const int i = t - 2;
      if (i >= 0) {
        if (i + PF < NSTEP) kf[(i + PF) % (PF + 1)] = kread(i + PF);
        const int kt = i % 2, c = i / 2;
        s_nxt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (PF + 1)], w.qf[c],
                                                            c == 0 ? f32x16{} : s_nxt[kt], 0, 0, 0);
      }
      if (t < NSTEP) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int v = t * PER + j;
          xs[t % 3][j] = fmaf(s_cur[v >> 4][v & 15], c_scale, -m_use);
        }
      }
      if (t >= 1 && t - 1 < NSTEP) {
#pragma unroll
        for (int j = 0; j < PER; ++j) xs[(t - 1) % 3][j] = fast_exp2(xs[(t - 1) % 3][j]);
      }
      if (i >= 0) {
#pragma unroll
        for (int j = 0; j < PER; j += 2) {
          const int v = i * PER + j;
          const int G = 2 * (v >> 4) + ((v & 15) >> 3), e = v & 7;
          pb[G][e] = (__bf16)xs[i % 3][j];
          pb[G][e + 1] = (__bf16)xs[i % 3][j + 1];
          const bf16x2 pr = {pb[G][e], pb[G][e + 1]};
          lp[(v >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, lp[(v >> 1) & 1], false);
        }
      }
      if (i >= 0) __builtin_amdgcn_sched_barrier(0);
    }
    w.l_run += lp[0] + lp[1];
  } else {
    if (live1) scores_tile<D, NW>(smem, kbuf_next, w, s_nxt);
    if (live0) exp_tile(s_cur, m_use, c_scale, pb, w.l_run);
  }
  return live0;
}

// Back half of pipeline step n: O^T += V(n)^T P(n)^T from V buffer vb.
template <int D, int NW>
__device__ __forceinline__ void step_back(char* smem, WaveState<D, NW>& w,
                                          const bf16x8 (&pb)[Bf16Cfg<D, NW>::NS / 8], int vb,
                                          bool live0) {
  using C = Bf16Cfg<D, NW>;
  constexpr int BC = C::BC;
  // O^T += V(n)^T P(n)^T: fragment j = (G = j / NDT, dt = j % NDT) is read
  // PF ops ahead, and consecutive ops accumulate into different d tiles
  if (live0) {
    constexpr int NJ = (BC / 16) * C::NDT;
    constexpr int PF = NJ >= 8 ? 4 : 2;
    unsigned vbase[C::NDT];
    const unsigned vl = (unsigned)(size_t)(lds_void_ptr)(smem + C::VB + vb * C::TILE);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) vbase[dt] = vl + w.vaddr[dt];
    // two 64-bit transposed reads per fragment: keys 16G .. 16G+7 and
    // 16G+8 .. 16G+15 of the fragment's d tile
    s16x8 vr[PF + 1];
    auto vread = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int off = (j / C::NDT) * 16 * C::ROWB;
      const s16x4 lo = lds_read_tr16<off>(vbase[j % C::NDT]);
      const s16x4 hi = lds_read_tr16<off + 8 * C::ROWB>(vbase[j % C::NDT]);
      vr[j % (PF + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    static_for<0, PF>([&](auto jc) { vread(jc); });
    // this phase is matrix-core bound: give it issue priority over the
    // other wave on the SIMD, whose exponentials fill the gaps
    __builtin_amdgcn_s_setprio(2);
    static_for<0, NJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + PF < NJ) vread(std::integral_constant<int, j + PF>{});
      // reads issued after fragment j's: those of fragments j+1 .. j+PF
      constexpr int later = 2 * ((j + PF < NJ ? j + PF : NJ - 1) - j);
      claim_lds<later>(vr[j % (PF + 1)]);
      bf16x8 vf;
      __builtin_memcpy(&vf, &vr[j % (PF + 1)], 16);
      constexpr int G = j / C::NDT, dt = j % C::NDT;
      w.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[G], w.oacc[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
  }
}

// One pipeline step.  PAR = n & 1: K(n+1) sits in K buffer PAR^1, V(n) in
// V buffer PAR; the copies go to K buffer PAR and V buffer PAR^1.
template <int D, int NW, int PAR>
__device__ __forceinline__ void pipeline_step(
    const AttnArgs& a, char* smem, WaveState<D, NW>& w, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
    Cursor& t0, Cursor& t1, Cursor& t2, int& vb,
    const Span& sp, long long wq_lo, long long wq_hi, int wrows, int col, int half, int b,
    int h, int HD2, int wave) {
  using C = Bf16Cfg<D, NW>;
  // copies of tile n+2: K first, so that waiting for it leaves V in flight
  const int vb2 = vb == 0 ? 2 : vb - 1;  // (vb + 2) % 3
  const bool copy2 = t2.blk < a.nblk;
  if (copy2) {
    const KVBlock& kb2 = a.blk[t2.blk];
    copy_tile<D, NW>(kb2.k, kb2.len, a.kv_rows_b, t2.t, b, h, a.Hkv, HD2, wave, w.voffk,
                 smem + C::KB + PAR * C::TILE);
    copy_tile<D, NW>(kb2.v, kb2.len, a.kv_rows_b, t2.t, b, h, a.Hkv, HD2, wave, w.voffv,
                 smem + C::VB + vb2 * C::TILE);
  }
  bf16x8 pb[C::NS / 8];
  const bool live0 = step_front<D, NW, PAR>(a, smem, w, s_cur, s_nxt, t0, t1, wq_lo, wq_hi,
                                            wrows, col, half, pb);
  step_back<D, NW>(smem, w, pb, vb, live0);
  // this wave's K(n+2) copy (and everything older) landed; V(n+2) may fly
  if (copy2) wait_vmcnt<C::DMA>();
  else wait_vmcnt<0>();
  pipeline_barrier();  // everyone's copies landed, everyone done reading
  t0 = t1;
  t1 = t2;
  t2 = cursor_next(a, sp, t2);
  vb = vb == 2 ? 0 : vb + 1;
}

// One step of the staggered form (8 waves, 256 query rows, one barrier per
// step).  Both groups run front(n) then back(n), but group 0 (waves 0-3)
// passes its barrier after back(n) and group 1 (waves 4-7) after front(n).
// Between two barriers the group-0 wave thus computes front(n), back(n)
// while its partner on the same SIMD computes back(n-1), front(n): one is
// in its vector-heavy half while the other is in its matrix-bound half.
// Group 0 copies whole tiles: K(n+2) into K(n)'s buffer and V(n+2) into
// V(n-2)'s (four V buffers, as group 1 reads V(n-1) during step n), and
// waits for its K(n+2) before its barrier.
template <int D, int PAR>
__device__ __forceinline__ void pp_step(
    const AttnArgs& a, char* smem, WaveState<D, 8>& w, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
    Cursor& t0, Cursor& t1, Cursor& t2, int& vb, const Span& sp, long long wq_lo,
    long long wq_hi, int wrows, int col, int half, int b, int h, int HD2, int gw, int grp,
    const int* voffk4, const int* voffv4) {
  using C = Bf16Cfg<D, 8>;
  const bool copy2 = grp == 0 && t2.blk < a.nblk;
  if (copy2) {
    const KVBlock& kb2 = a.blk[t2.blk];
    copy_tile<D, 4>(kb2.k, kb2.len, a.kv_rows_b, t2.t, b, h, a.Hkv, HD2, gw, voffk4,
                    smem + C::KB + PAR * C::TILE);
    copy_tile<D, 4>(kb2.v, kb2.len, a.kv_rows_b, t2.t, b, h, a.Hkv, HD2, gw, voffv4,
                    smem + C::VB + ((vb + 2) & 3) * C::TILE);
  }
  bf16x8 pb[C::NS / 8];
  const bool live0 = step_front<D, 8, PAR>(a, smem, w, s_cur, s_nxt, t0, t1, wq_lo, wq_hi,
                                           wrows, col, half, pb);
  if (grp == 1) pipeline_barrier();
  step_back<D, 8>(smem, w, pb, vb, live0);
  if (grp == 0) {
    // this wave's K(n+2) copy (and everything older) landed; V(n+2) may fly
    if (copy2) wait_vmcnt<Bf16Cfg<D, 4>::DMA>();
    else wait_vmcnt<0>();
    pipeline_barrier();
  }
  t0 = t1;
  t1 = t2;
  t2 = cursor_next(a, sp, t2);
  vb = (vb + 1) & 3;
}

// One (batch, head, query tile) over tiles [lo, hi) of its visited-tile
// sequence, shared by the 32-row-per-wave kernels; PP selects the staggered
// form (NW = 8 only).  slot < 0: the output rows of the tile; otherwise the
// split partial slot (see AttnArgs).
template <int D, int NW, bool PP>
__device__ __forceinline__ void attn_bf16_tile(const AttnArgs& a, char* smem, int b, int h,
                                               int qt, int lo, int hi, long long slot) {
  using C = Bf16Cfg<D, NW>;
  static_assert(!PP || NW == 8, "the staggered form pairs waves w and w+4 on one SIMD");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int row0 = qt * C::BR;
  const int rows_here = min(C::BR, a.Sq - row0);
  Span sp{qpos(a, row0 + rows_here - 1), a.nblk, 0};
  if (hi != INT_MAX) {
    const Cursor e = seq_pos(a, sp.q_hi, hi);
    sp.end_blk = e.blk;
    sp.end_t = e.t;
  }
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = qpos(a, wrow0);
  const long long wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;
  const int HD2 = a.Hkv * D * 2;  // bytes between consecutive key rows
  const int hk = h / (a.H / a.Hkv);  // K/V head of this query head

  WaveState<D, NW> w;
  {
    const int r = wrow0 + col;
    const __bf16* qp = (const __bf16*)a.q + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
      w.qf[c] = r < a.Sq ? *(const bf16x8*)(qp + 16 * c + 8 * half) : bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int p = (wave * C::DMA + i) * 64 + lane;  // physical 16B chunk in the tile
    const int r = p / C::CHUNKS, pc = p % C::CHUNKS;
    w.voffk[i] = r * HD2 + swz_k<D>(r, pc) * 16;
    w.voffv[i] = r * HD2 + swz_v<D>(r, pc) * 16;
  }
#pragma unroll
  for (int c = 0; c < C::NC; ++c) w.kaddr[c] = col * C::ROWB + swz_k<D>(col, 2 * c + half) * 16;
  {
    const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
    const int kl = 4 * half + e;  // supplier row within a 16-key group
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
      w.vaddr[dt] = kl * C::ROWB + swz_v<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) w.oacc[i] = f32x16{};
  w.m_ref = -INFINITY;
  w.m_true = -INFINITY;
  w.l_run = 0.0f;

  // staggered form: group of the wave, its index in the group and, for
  // group 0, the copy offsets of whole tiles over four waves
  const int grp = wave >> 2, gw = wave & 3;
  int voffk4[PP ? Bf16Cfg<D, 4>::DMA : 1], voffv4[PP ? Bf16Cfg<D, 4>::DMA : 1];
  if constexpr (PP) {
#pragma unroll
    for (int i = 0; i < Bf16Cfg<D, 4>::DMA; ++i) {
      const int p = (gw * Bf16Cfg<D, 4>::DMA + i) * 64 + lane;
      const int r = p / C::CHUNKS, pc = p % C::CHUNKS;
      voffk4[i] = r * HD2 + swz_k<D>(r, pc) * 16;
      voffv4[i] = r * HD2 + swz_v<D>(r, pc) * 16;
    }
  }

  // prologue: K(0), V(0), K(1) into K0, V0, K1; scores of tile 0
  Cursor t0 = cursor_first(a, sp, lo);
  Cursor t1 = cursor_next(a, sp, t0);
  Cursor t2 = cursor_next(a, sp, t1);
  f32x16 sA[2], sB[2];
  if (t0.blk < a.nblk) {
    const KVBlock& kb = a.blk[t0.blk];
    copy_tile<D, NW>(kb.k, kb.len, a.kv_rows_b, t0.t, b, hk, a.Hkv, HD2, wave, w.voffk,
                     smem + C::KB);
    copy_tile<D, NW>(kb.v, kb.len, a.kv_rows_b, t0.t, b, hk, a.Hkv, HD2, wave, w.voffv,
                     smem + C::VB);
  }
  if (t1.blk < a.nblk) {
    const KVBlock& kb = a.blk[t1.blk];
    copy_tile<D, NW>(kb.k, kb.len, a.kv_rows_b, t1.t, b, hk, a.Hkv, HD2, wave, w.voffk,
                     smem + C::KB + C::TILE);
    copy_tile<D, NW>(kb.v, kb.len, a.kv_rows_b, t1.t, b, hk, a.Hkv, HD2, wave, w.voffv,
                     smem + C::VB + C::TILE);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t0.blk < a.nblk) {
    const long long kp0 = a.blk[t0.blk].k_pos0 + (long long)t0.t * C::BC;
    if (wrows > 0 && !(a.causal && kp0 > wq_hi)) scores_tile<D, NW>(smem, C::KB, w, sA);
  }
  __syncthreads();  // K buffer 0 is free for K(2)

  int vb = 0;  // V buffer of tile n
  if constexpr (PP) {
    while (t0.blk < a.nblk) {
      pp_step<D, 0>(a, smem, w, sA, sB, t0, t1, t2, vb, sp, wq_lo, wq_hi, wrows, col, half, b,
                    hk, HD2, gw, grp, voffk4, voffv4);
      if (t0.blk >= a.nblk) break;
      pp_step<D, 1>(a, smem, w, sB, sA, t0, t1, t2, vb, sp, wq_lo, wq_hi, wrows, col, half, b,
                    hk, HD2, gw, grp, voffk4, voffv4);
    }
  } else {
    while (t0.blk < a.nblk) {
      pipeline_step<D, NW, 0>(a, smem, w, sA, sB, t0, t1, t2, vb, sp, wq_lo, wq_hi, wrows,
                              col, half, b, hk, HD2, wave);
      if (t0.blk >= a.nblk) break;
      pipeline_step<D, NW, 1>(a, smem, w, sB, sA, t0, t1, t2, vb, sp, wq_lo, wq_hi, wrows,
                              col, half, b, hk, HD2, wave);
    }
  }

  // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
  const float l_tot = pair_sum(w.l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int r = wrow0 + col;
  if (wrows > 0 && r < a.Sq) {
    // output row (b, r, h), or row r - row0 of the split partial slot
    const long long so = slot < 0 ? ((long long)b * a.Sq + r) * a.H + h
                                  : slot * C::BR + (r - row0);
    const long long ro = so * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const float x0 = w.oacc[dt][4 * g + 0] * inv, x1 = w.oacc[dt][4 * g + 1] * inv;
        const float x2 = w.oacc[dt][4 * g + 2] * inv, x3 = w.oacc[dt][4 * g + 3] * inv;
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
      const bool seen = l_tot > 0.0f;
      if (a.lse) a.lse[so] = seen ? (w.m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (a.m_out) a.m_out[so] = seen ? w.m_true * kLn2 : -INFINITY;
      if (a.l_out) a.l_out[so] = seen ? l_tot * fast_exp2(w.m_ref - w.m_true) : 0.0f;
    }
  }
}

// Kernel body shared by the 32-row-per-wave kernels: one query tile over its
// whole visited sequence, or (SPLIT) one run of it.
template <int D, int NW, bool PP, bool SPLIT = false>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a, char* smem) {
  using C = Bf16Cfg<D, NW>;
  if constexpr (SPLIT) {
    const int ns = a.nsplit;
    const int j = (int)blockIdx.x % ns;
    const int tile = (int)blockIdx.x / ns;  // (b*H + h)*n_qtiles + qt
    const int qt = tile % a.n_qtiles, bh = tile / a.n_qtiles;
    const int row_hi = min((qt + 1) * C::BR, a.Sq) - 1;
    const long long q_hi = qpos(a, row_hi);
    int total = 0;
    for (int bi = 0; bi < a.nblk; ++bi) total += tiles_of<64>(a, bi, q_hi);
    const int lo = (int)((long long)total * j / ns), hi = (int)((long long)total * (j + 1) / ns);
    attn_bf16_tile<D, NW, PP>(a, smem, bh / a.H, bh % a.H, qt, lo, hi, (long long)tile * ns + j);
  } else {
    int b, h, qt;
    tile_coords(a, b, h, qt);
    attn_bf16_tile<D, NW, PP>(a, smem, b, h, qt, 0, INT_MAX, -1);
  }
}
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, NW>::LDS];
  attn_bf16_body<D, NW, false>(a, smem);
}

// The split ring on the 128-row kernel (AttnArgs.nsplit > 1).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16_split(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, 4>::LDS];
  attn_bf16_body<D, 4, false, true>(a, smem);
}

// Staggered form: 8 waves x 32 query rows, one workgroup per CU, two K and
// four V buffers.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16_pp(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, 8>::LDS + Bf16Cfg<D, 8>::TILE];
  attn_bf16_body<D, 8, true>(a, smem);
}

// ---------------------------------------------------------------------------
// bf16 kernel, 64 query rows per wave
// ---------------------------------------------------------------------------
// Same arithmetic as ring_attn_bf16, but each wave owns 64 query rows (two
// 32-row column blocks cb = 0, 1) and runs alone on its SIMD with the whole
// register file (512 registers; the O^T accumulators live in AGPRs).  Every
// K or V fragment read from LDS then feeds two matrix ops instead of one,
// which halves LDS read traffic per FLOP, and a workgroup of four waves
// covers 256 query rows, which halves the HBM/L2 -> LDS copies per FLOP.
//
// K/V move through LDS in stages of 64 keys; the wave computes in sub-tiles
// of 32 keys.  Sub-step j (two per stage) runs
//   phase B: S^T(j+1) = K(j+1) Q^T on the matrix cores, interleaved with
//            the exponentials of tile j and their bf16 copy P(j);
//   phase C: O^T += V(j)^T P(j)^T, interleaved with the denominator of P(j),
//            the mask and row max of S(j+1), the choice of its reference max
//            and the scaled, shifted scores of S(j+1).
// A rescale of O and l forced by a new reference max (rare, see the lazy
// reference above) is applied at the start of the next sub-step, after the
// P V products of the old reference were issued.
//
// Stage pipeline (n = stage of the iteration): LDS holds K(n), K(n+1), V(n);
// the iteration issues the copies of K(n+3) and V(n+2) and, before its
// closing barrier, waits for those of K(n+2) and V(n+1), issued one
// iteration earlier: every copy has two iterations to land.  Four K and
// three V buffers (112 KiB at D = 128).
template <int D>
struct W64Cfg {
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int WR = 64;                   // query rows per wave
  static constexpr int BR = NW * WR;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per LDS stage
  static constexpr int ROWB = D * 2;              // bytes per key row in LDS
  static constexpr int TILE = BC * ROWB;          // one K or V stage
  static constexpr int NKB = 4, NVB = 3;          // stage buffers
  static constexpr int KB = 0, VB = NKB * TILE;
  static constexpr int LDS = (NKB + NVB) * TILE;
  static constexpr int CHUNKS = D / 8;
  static constexpr int DMA = TILE / 1024 / NW;    // 1 KiB copies per wave per stage
  static constexpr int NC = D / 16;               // k-steps of S^T
  static constexpr int NDT = D / 32;              // 32-row d tiles of O^T
  static constexpr int KPF = 4;                   // K fragment lead (fragments)
  static constexpr int VPF = 3;                   // V fragment lead (fragments)
};

// A 64-key stage of the visited sequence with everything the loop needs
// about it.  The kernel arguments (the block table) are read only when the
// sequence enters a new block; inside a block a stage advances by pointer
// arithmetic.  Positions are 32-bit here (the host routes longer sequences
// to the other kernels).
struct Stage {
  int blk;           // visited block, a.nblk once past the end
  int t, n;          // stage t of the n this workgroup visits in the block
  int kp;            // global position of the stage's first key
  int rows;          // rows of the block from that key on (>= 64: a full stage)
  const char* k;     // K of this (batch, head) from that key on
  const char* v;     // V likewise
};

__device__ __forceinline__ Stage stage_enter(const AttnArgs& a, int blk, long long q_hi, int b,
                                             int h, int D2, int HD2) {
  Stage s;
  s.blk = blk;
  s.t = 0;
  s.n = 0;
  while (s.blk < a.nblk && (s.n = tiles_of<64>(a, s.blk, q_hi)) == 0) ++s.blk;
  s.kp = 0;
  s.rows = 0;
  s.k = s.v = nullptr;
  if (s.blk < a.nblk) {
    const KVBlock& kb = a.blk[s.blk];
    const long long off = (long long)b * a.kv_rows_b * HD2 + (long long)h * D2;
    s.kp = (int)kb.k_pos0;
    s.rows = kb.len;
    s.k = (const char*)kb.k + off;
    s.v = (const char*)kb.v + off;
  }
  return s;
}

__device__ __forceinline__ Stage stage_next(const AttnArgs& a, Stage s, long long q_hi, int b,
                                            int h, int D2, int HD2) {
  if (s.blk >= a.nblk) return s;
  if (++s.t < s.n) {
    s.kp += 64;
    s.rows -= 64;
    s.k += 64LL * HD2;
    s.v += 64LL * HD2;
    return s;
  }
  return stage_enter(a, s.blk + 1, q_hi, b, h, D2, HD2);
}

// Copy one stage (64 key rows of K or V from src) into LDS at dst; each wave
// copies its share.  Rows past the block's end come back as zeros from the
// buffer range check.  lds_wave is this wave's first 1 KiB slot (uniform).
template <int D>
__device__ __forceinline__ void copy_stage(const char* src, int rows, int HD2, const int* voff,
                                           unsigned dst) {
  using C = W64Cfg<D>;
  const int nrec = (min(rows, C::BC) - 1) * HD2 + D * 2;
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, nrec, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < C::DMA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(size_t)(dst + i * 1024), 16,
                                             voff[i], 0, 0, 0);
}

// A stage copy to be issued during a sub-step, one 1 KiB instruction at a
// time between matrix ops, so that the wave's vector-memory issue hides
// under them (issued back to back, the copies stall a wave that has no
// other to cover for it).
struct StageCopy {
  __amdgpu_buffer_rsrc_t rs;
  const int* voff;
  unsigned dst;    // this wave's first 1 KiB slot
  bool on;
};

template <int D>
__device__ __forceinline__ StageCopy stage_copy(const char* src, int rows, int HD2,
                                                const int* voff, unsigned dst, bool on) {
  using C = W64Cfg<D>;
  StageCopy c;
  const int nrec = (min(rows, C::BC) - 1) * HD2 + D * 2;
  c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, nrec, kRsrcWord3);
  c.voff = voff;
  c.dst = dst;
  c.on = on;
  return c;
}

__device__ __forceinline__ void stage_copy_part(const StageCopy& c, int i) {
  if (c.on)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (lds_void_ptr)(size_t)(c.dst + i * 1024), 16,
                                             c.voff[i], 0, 0, 0);
}

// One 32-key sub-tile as this wave sees it.
struct Sub {
  bool mask;       // some (row, key) pair of it must be masked (all, if dead)
  int kp;          // global position of its first key
  int klim;        // keys [0, klim) exist, are not padding and may be visible
};

__device__ __forceinline__ Sub sub_info(const Stage& st, int sub, bool causal, int valid_len,
                                        int wq_lo, int wq_hi, bool wave_live) {
  Sub s{true, 0, 0};  // dead: every pair masked
  if (!wave_live || st.n == 0) return s;
  s.kp = st.kp + 32 * sub;
  int lim = min(st.rows - 32 * sub, valid_len - s.kp);
  lim = min(lim, 32);
  const bool live = lim > 0 && !(causal && s.kp > wq_hi);
  s.klim = live ? lim : 0;
  s.mask = !live || lim < 32 || (causal && s.kp + 31 > wq_lo);
  return s;
}

template <int D>
struct W64State {
  using C = W64Cfg<D>;
  bf16x8 qf[2][C::NC];     // Q^T fragments of the two column blocks
  f32x16 oacc[2][C::NDT];  // O^T accumulators (unnormalised u)
  float m_ref[2];          // reference max (base 2), -inf before any key
  float m_true[2];         // exact running max (base 2)
  float m_use[2];          // shift applied to the scores in flight
  float alpha[2];          // pending rescale factor of O and l
  float l_run[2];          // this lane's half of sum of bf16(2^(s - m_ref))
  int kaddr[C::NC];
  int vaddr[C::NDT];
  int voffk[C::DMA];
  int voffv[C::DMA];
};

// Mask of S^T for column block cb of a sub-tile: key j (0..31) of lane
// (col, half) at register v is 8*(v/4) + v%4 + 4*half; it is masked when
// j >= klim or, causal, when its position exceeds the query's.
__device__ __forceinline__ void mask_sub(f32x16& s, const Sub& st, bool causal, int wq_lo,
                                         int cb, int col, int half) {
  int t = st.klim - 1 - 4 * half;
  if (causal) {
    const int dc = min(64, max(-64, wq_lo + 32 * cb - st.kp));
    t = min(t, max(-1, dc + col - 4 * half));
  }
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (8 * (v >> 2) + (v & 3) > t) s[v] = -INFINITY;
}

// max(a, b, c) in one instruction.  Written as assembly because the
// compiler's fmaxf first quiets signalling NaNs (an extra v_max per operand)
// for values it cannot prove canonical, such as matrix-core results.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// S^T = K Q^T products with the accumulator in VGPRs, written as assembly.
// The compiler would put every matrix-core accumulator of this kernel in
// AGPRs (it needs more than 256 registers), and the scores would then have
// to be copied out before any vector instruction could read them.  As the
// compiler does not see these as matrix ops, the reader of a result must
// first let the matrix pipe drain (mfma_results_ready); dependent products
// on the same accumulator need no wait.
__device__ __forceinline__ void mfma_v_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 16 wait states: more than an 8-pass matrix op needs before a vector
// instruction may read its result.
__device__ __forceinline__ void mfma_results_ready() {
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
}

__device__ __forceinline__ float max16(const f32x16& s) {
  float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, s[15]));
}

// Row max of the (masked) scores of the next sub-tile and the choice of
// its reference ([RA] §3.2 with the lazy reference): sets m_use and, when
// the reference moves, alpha and the returned flag.
template <int D>
__device__ __forceinline__ bool decide(W64State<D>& w, const float (&mlane)[2], float c_scale) {
  float mx[2];
  bool need[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    mx[cb] = pair_max(mlane[cb]) * c_scale;
    w.m_true[cb] = fmaxf(w.m_true[cb], mx[cb]);
    need[cb] = mx[cb] > w.m_ref[cb] + kRescaleSlack;
  }
  const bool any = __builtin_amdgcn_ballot_w64(need[0] || need[1]) != 0;
  if (any) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      w.alpha[cb] = need[cb] ? fast_exp2(w.m_ref[cb] - mx[cb]) : 1.0f;
      w.m_ref[cb] = need[cb] ? mx[cb] : w.m_ref[cb];
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) w.m_use[cb] = w.m_ref[cb] == -INFINITY ? 0.0f : w.m_ref[cb];
  return any;
}

// acc *= alpha for an accumulator held in AGPRs.  The product is formed in
// inline assembly on each AGPR in place, so the accumulator never has to
// leave the AGPR file (vector ALU instructions cannot name AGPRs).
__device__ __forceinline__ void scale_agpr(f32x16& acc, float alpha) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = acc[v], t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(alpha));
    acc[v] = x;
  }
}

template <int D>
__device__ __forceinline__ void apply_rescale(W64State<D>& w) {
  using C = W64Cfg<D>;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    w.l_run[cb] *= w.alpha[cb];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) scale_agpr(w.oacc[cb][i], w.alpha[cb]);
  }
}

// S^T of one sub-tile (no interleave): K rows at LDS offset kofs; results
// readable after mfma_results_ready().
template <int D>
__device__ __forceinline__ void scores_sub(char* smem, int kofs, const W64State<D>& w,
                                           f32x16 (&s)[2]) {
  using C = W64Cfg<D>;
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    const bf16x8 kf = *(const bf16x8*)(smem + kofs + w.kaddr[c]);
    if (c == 0) {
      mfma_v_first(s[0], kf, w.qf[0][c]);
      mfma_v_first(s[1], kf, w.qf[1][c]);
    } else {
      mfma_v_acc(s[0], kf, w.qf[0][c]);
      mfma_v_acc(s[1], kf, w.qf[1][c]);
    }
  }
}

// One sub-step.  s_cur holds the raw scores of sub-tile j (cur, masked,
// reference already chosen), s_nxt receives S^T of sub-tile j+1 (nxt) from
// the K rows at LDS offset kofs; P(j) V(j) uses the V rows at LDS offset
// vofs (32 keys).  The code has no branch on liveness: a sub-tile that is
// dead for this wave is masked entirely (its scores become -inf, its
// weights 0), which keeps the O^T accumulators in one register class across
// the loop.  The V rows of cur always belong to a copied stage (zero-filled
// past a block's end), so 0 * V stays 0; the K rows of a dead nxt may be
// stale, but are always rows of a copied stage, and the mask replaces every
// score they produce.
//
// Operand reads run ahead across phase boundaries: the first K fragments of
// a sub-step are read (into kf) during the previous sub-step's last matrix
// ops, the first V fragments of phase C during phase B's last ones.
template <int D>
__device__ __forceinline__ void w64_substep(const AttnArgs& a, char* smem, W64State<D>& w,
                                            f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                            bf16x8 (&kf)[W64Cfg<D>::KPF + 1], const Sub& nxt,
                                            int kofs, int kofs_next, unsigned vofs,
                                            const StageCopy& cp, bool& pending, int wq_lo,
                                            int col, int half) {
  using C = W64Cfg<D>;
  constexpr int NF = 2 * C::NDT;         // V fragments (G, dt) of the sub-tile
  constexpr int VPF = C::VPF;
  const float c_scale = a.scale_log2;
  if (pending) {  // the reference moved when cur's reference was chosen
    apply_rescale(w);
    pending = false;
  }
  s16x8 vr[VPF + 1];
  auto vread = [&](auto fc) {
    constexpr int f = decltype(fc)::value;
    constexpr int off = (f / C::NDT) * 16 * C::ROWB;
    const unsigned base = vofs + w.vaddr[f % C::NDT];
    const s16x4 lo = lds_read_tr16<off>(base);
    const s16x4 hi = lds_read_tr16<off + 8 * C::ROWB>(base);
    vr[f % (VPF + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // ---- phase B: S^T(nxt) alongside the weights P(cur) ----
  // The weights go through three stages one matrix op apart, so that no
  // vector instruction waits on the one just before it: pair x (scores 2x,
  // 2x+1: block x / 8, registers 2 (x % 8), +1) is scaled and shifted
  // (t = s * scale - m_use) at op x / PPS, exponentiated at the next op and
  // rounded to bf16 at the one after; the last pairs finish under the first
  // ops of phase C.
  constexpr int NSTEP = 2 * C::NC;       // phase B matrix ops (k-step c, block cb)
  constexpr int PPS = 16 / NSTEP;        // weight pairs per op
  bf16x8 pb[2][2];
  float tq[3][PPS][2], eq[3][PPS][2];
  auto w_stage = [&](auto ic) {  // the weight stages that belong to op i
    constexpr int i = decltype(ic)::value;
    static_for<0, PPS>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      // (each stage's results are pinned to its op: left alone, the
      // compiler sinks the whole chain to the first use in phase C)
      if constexpr (i >= 2 && i - 2 < NSTEP) {  // round to bf16
        constexpr int x = (i - 2) * PPS + u, eb = x >> 3, v = 2 * (x & 7);
        pb[eb][v >> 3][v & 7] = (__bf16)eq[(i - 2) % 3][u][0];
        pb[eb][v >> 3][(v & 7) + 1] = (__bf16)eq[(i - 2) % 3][u][1];
        asm volatile("" ::"v"(pb[eb][v >> 3]));
      }
      if constexpr (i >= 1 && i - 1 < NSTEP) {  // exponentiate
        eq[(i - 1) % 3][u][0] = fast_exp2(tq[(i - 1) % 3][u][0]);
        eq[(i - 1) % 3][u][1] = fast_exp2(tq[(i - 1) % 3][u][1]);
        asm volatile("" ::"v"(eq[(i - 1) % 3][u][0]), "v"(eq[(i - 1) % 3][u][1]));
      }
      if constexpr (i < NSTEP) {  // scale and shift
        constexpr int x = i * PPS + u, eb = x >> 3, v = 2 * (x & 7);
        tq[i % 3][u][0] = fmaf(s_cur[eb][v], c_scale, -w.m_use[eb]);
        tq[i % 3][u][1] = fmaf(s_cur[eb][v + 1], c_scale, -w.m_use[eb]);
        asm volatile("" ::"v"(tq[i % 3][u][0]), "v"(tq[i % 3][u][1]));
      }
    });
  };
  {
    constexpr int PF = C::KPF;
    auto kread = [&](int c) -> bf16x8 { return *(const bf16x8*)(smem + kofs + w.kaddr[c]); };
    static_for<0, NSTEP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int c = i >> 1, cb = i & 1;
      if constexpr (cb == 0 && c + PF < C::NC) kf[(c + PF) % (PF + 1)] = kread(c + PF);
      if constexpr (c == 0) mfma_v_first(s_nxt[cb], kf[c % (PF + 1)], w.qf[cb][c]);
      else mfma_v_acc(s_nxt[cb], kf[c % (PF + 1)], w.qf[cb][c]);
      w_stage(ic);
      // the last K fragment is in registers: start phase C's V reads
      if constexpr (i == NSTEP - 2) static_for<0, VPF>([&](auto fc) { vread(fc); });
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  mfma_results_ready();
  if (nxt.mask) {  // diagonal, ragged or dead sub-tile
    mask_sub(s_nxt[0], nxt, a.causal, wq_lo, 0, col, half);
    mask_sub(s_nxt[1], nxt, a.causal, wq_lo, 1, col, half);
  }
  // ---- phase C: O^T += V(cur)^T P(cur)^T alongside the max of nxt (first
  // half of the ops) and the denominator of P(cur) (second half) ----
  {
    constexpr int NJ = 2 * NF;           // matrix ops (fragment, block cb)
    constexpr int PF = VPF;
    float lp[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    float mxp[2] = {-INFINITY, -INFINITY};  // this lane's max of nxt per block
    auto pv_op = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int f = j / 2, cb = j % 2;
      if constexpr (cb == 0) {
        if constexpr (f + PF < NF) vread(std::integral_constant<int, f + PF>{});
        constexpr int later = 2 * ((f + PF < NF ? f + PF : NF - 1) - f);
        claim_lds<later>(vr[f % (PF + 1)]);
      }
      bf16x8 vf;
      __builtin_memcpy(&vf, &vr[f % (PF + 1)], 16);
      constexpr int G = f / C::NDT, dt = f % C::NDT;
      w.oacc[cb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[cb][G], w.oacc[cb][dt],
                                                               0, 0, 0);
    };
    constexpr int NH = NJ / 2;
    static_for<0, NH>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      pv_op(jc);
      // the last weight pairs of cur: needed from op 2 NDT + 1 on
      if constexpr (j < 2) w_stage(std::integral_constant<int, NSTEP + j>{});
      if constexpr (j == 1)
        asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]));
      if constexpr ((j & 1) && (j >> 1) < C::DMA) stage_copy_part(cp, j >> 1);
      // 32 / NH scores of nxt into its row max (score x: block x / 16)
      static_for<0, 32 / NH / 2>([&](auto yc) {
        constexpr int x = j * 32 / NH + 2 * decltype(yc)::value;
        constexpr int mb = x >> 4, q = x & 15;
        mxp[mb] = vmax3(mxp[mb], s_nxt[mb][q], s_nxt[mb][q + 1]);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    pending = decide(w, mxp, c_scale);
    static_for<NH, NJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      pv_op(jc);
      // 16 / NH bf16 pairs of P(cur) into the denominator (pair x: block
      // x / 8, fragment (x / 4) % 2, elements 2 (x % 4), +1)
      static_for<(j - NH) * 16 / NH, (j - NH + 1) * 16 / NH>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        constexpr int eb = x >> 3, G2 = (x >> 2) & 1, e = 2 * (x & 3);
        const bf16x2 pr = {pb[eb][G2][e], pb[eb][G2][e + 1]};
        lp[eb][x & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, lp[eb][x & 1], false);
      });
      // every V read is claimed: start the next sub-step's K reads
      if constexpr (j == NJ - 2) {
#pragma unroll
        for (int c = 0; c < C::KPF; ++c)
          kf[c] = *(const bf16x8*)(smem + kofs_next + w.kaddr[c]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // keep the denominator updates under the matrix ops as well
    asm volatile("" ::"v"(lp[0][0]), "v"(lp[0][1]), "v"(lp[1][0]), "v"(lp[1][1]));
    w.l_run[0] += lp[0][0] + lp[0][1];
    w.l_run[1] += lp[1][0] + lp[1][1];
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ring_attn_bf16_w64(const AttnArgs a) {
  using C = W64Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  int b, h, qt;
  tile_coords(a, b, h, qt);
  const int row0 = qt * C::BR;
  const int rows_here = min(C::BR, a.Sq - row0);
  const long long q_hi = qpos(a, row0 + rows_here - 1);
  const int wrow0 = row0 + wave * C::WR;
  const int wrows = min(C::WR, a.Sq - wrow0);
  const bool wave_live = wrows > 0;
  const int wq_lo = (int)qpos(a, wrow0);
  const int wq_hi = wq_lo + wrows - 1;
  const int valid_len = a.valid_len > 0x7fffffffLL ? 0x7fffffff : (int)a.valid_len;
  const bool causal = a.causal != 0;
  const long long HD = (long long)a.H * D;
  const int D2 = D * 2;
  const int HD2 = a.Hkv * D2;
  const int hk = h / (a.H / a.Hkv);  // K/V head of this query head

  W64State<D> w;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = wrow0 + 32 * cb + col;
    const __bf16* qp = (const __bf16*)a.q + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int c = 0; c < C::NC; ++c)
      w.qf[cb][c] = r < a.Sq ? *(const bf16x8*)(qp + 16 * c + 8 * half) : bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int p = (wave * C::DMA + i) * 64 + lane;
    const int r = p / C::CHUNKS, pc = p % C::CHUNKS;
    w.voffk[i] = r * HD2 + swz_k<D>(r, pc) * 16;
    w.voffv[i] = r * HD2 + swz_v<D>(r, pc) * 16;
  }
#pragma unroll
  for (int c = 0; c < C::NC; ++c) w.kaddr[c] = col * C::ROWB + swz_k<D>(col, 2 * c + half) * 16;
  {
    const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
    const int kl = 4 * half + e;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
      w.vaddr[dt] = kl * C::ROWB + swz_v<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) w.oacc[cb][i] = f32x16{};
    w.m_ref[cb] = -INFINITY;
    w.m_true[cb] = -INFINITY;
    w.m_use[cb] = 0.0f;
    w.alpha[cb] = 1.0f;
    w.l_run[cb] = 0.0f;
  }
  const unsigned smem_lds = (unsigned)(size_t)(lds_void_ptr)smem;
  // this wave's 1 KiB copy slots within a stage buffer
  const unsigned kdst0 = smem_lds + C::KB + wave * C::DMA * 1024;
  const unsigned vdst0 = smem_lds + C::VB + wave * C::DMA * 1024;

  // prologue: stages 0..2 of K, 0..1 of V; scores of sub-tile 0
  Stage t0 = stage_enter(a, 0, q_hi, b, hk, D2, HD2);
  Stage t1 = stage_next(a, t0, q_hi, b, hk, D2, HD2);
  Stage t2 = stage_next(a, t1, q_hi, b, hk, D2, HD2);
  Stage t3 = stage_next(a, t2, q_hi, b, hk, D2, HD2);
  if (t0.blk < a.nblk) {
    copy_stage<D>(t0.k, t0.rows, HD2, w.voffk, kdst0);
    copy_stage<D>(t0.v, t0.rows, HD2, w.voffv, vdst0);
  }
  if (t1.blk < a.nblk) {
    copy_stage<D>(t1.k, t1.rows, HD2, w.voffk, kdst0 + C::TILE);
    copy_stage<D>(t1.v, t1.rows, HD2, w.voffv, vdst0 + C::TILE);
  }
  if (t2.blk < a.nblk) copy_stage<D>(t2.k, t2.rows, HD2, w.voffk, kdst0 + 2 * C::TILE);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sA[2], sB[2];
  bool pending = false;
  if (t0.blk < a.nblk) {
    const Sub s0 = sub_info(t0, 0, causal, valid_len, wq_lo, wq_hi, wave_live);
    scores_sub<D>(smem, C::KB, w, sA);
    mfma_results_ready();
    if (s0.mask) {
      mask_sub(sA[0], s0, causal, wq_lo, 0, col, half);
      mask_sub(sA[1], s0, causal, wq_lo, 1, col, half);
    }
    const float ml[2] = {max16(sA[0]), max16(sA[1])};
    decide(w, ml, a.scale_log2);  // nothing accumulated yet: no rescale
  }

  // K fragments of the first sub-step (stage 0, sub-tile 1)
  bf16x8 kf[C::KPF + 1];
#pragma unroll
  for (int c = 0; c < C::KPF; ++c) kf[c] = *(const bf16x8*)(smem + C::KB + 32 * C::ROWB + w.kaddr[c]);
  int kb0 = 0, vb0 = 0;  // K / V buffer of stage n
  while (t0.blk < a.nblk) {
    // copies of V(n+2) and K(n+3) into the buffers stage n-1 released,
    // issued piecewise during the two sub-steps
    const bool ck = t3.blk < a.nblk, cv = t2.blk < a.nblk;
    const int vbuf = vb0 == 0 ? 2 : vb0 - 1;  // (n + 2) % 3
    const StageCopy cpv =
        stage_copy<D>(t2.v, t2.rows, HD2, w.voffv, vdst0 + vbuf * C::TILE, cv);
    const StageCopy cpk =
        stage_copy<D>(t3.k, t3.rows, HD2, w.voffk, kdst0 + ((kb0 + 3) & 3) * C::TILE, ck);
    const Sub s01 = sub_info(t0, 1, causal, valid_len, wq_lo, wq_hi, wave_live);
    const Sub s10 = sub_info(t1, 0, causal, valid_len, wq_lo, wq_hi, wave_live);
    const int k_n = C::KB + kb0 * C::TILE;
    // past the last stage nxt is dead: point it at rows that were copied
    const int k_n1 = t1.blk < a.nblk ? C::KB + ((kb0 + 1) & 3) * C::TILE : k_n;
    const unsigned v_n = smem_lds + C::VB + vb0 * C::TILE;
    // sub-step 2n: S(stage n, sub 1), P V of (stage n, sub 0)
    w64_substep<D>(a, smem, w, sA, sB, kf, s01, k_n + 32 * C::ROWB, k_n1, v_n, cpv, pending,
                   wq_lo, col, half);
    // sub-step 2n+1: S(stage n+1, sub 0), P V of (stage n, sub 1); its
    // K(n+1) stays resident across the barrier, so the next sub-step's
    // (stage n+1, sub-tile 1) K reads may start before it
    w64_substep<D>(a, smem, w, sB, sA, kf, s10, k_n1, k_n1 + 32 * C::ROWB,
                   v_n + 2 * 16 * C::ROWB, cpk, pending, wq_lo, col, half);
    // this wave's copies of K(n+2) and V(n+1) landed; K(n+3), V(n+2) may fly
    if (ck) wait_vmcnt<2 * C::DMA>();
    else if (cv) wait_vmcnt<C::DMA>();
    else wait_vmcnt<0>();
    // every LDS read of K(n) and V(n) has been consumed by a matrix op; the
    // K(n+1) reads still in flight target a buffer no copy overwrites next
    asm volatile("s_barrier" ::: "memory");
    t0 = t1;
    t1 = t2;
    t2 = t3;
    t3 = stage_next(a, t3, q_hi, b, hk, D2, HD2);
    kb0 = (kb0 + 1) & 3;
    vb0 = vb0 == 2 ? 0 : vb0 + 1;
  }
  if (pending) apply_rescale(w);

  // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l_tot = pair_sum(w.l_run[cb]);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int r = wrow0 + 32 * cb + col;
    if (r >= a.Sq) continue;
    const long long ro = ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const float x0 = w.oacc[cb][dt][4 * g + 0] * inv, x1 = w.oacc[cb][dt][4 * g + 1] * inv;
        const float x2 = w.oacc[cb][dt][4 * g + 2] * inv, x3 = w.oacc[cb][dt][4 * g + 3] * inv;
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
      if (a.lse) a.lse[so] = seen ? (w.m_ref[cb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (a.m_out) a.m_out[so] = seen ? w.m_true[cb] * kLn2 : -INFINITY;
      if (a.l_out) a.l_out[so] = seen ? l_tot * fast_exp2(w.m_ref[cb] - w.m_true[cb]) : 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel, producer / consumer waves
// ---------------------------------------------------------------------------
// Eight waves per workgroup = four (producer, consumer) pairs, each pair
// owning 64 query rows, the pair's two waves sharing one SIMD.  The producer
// holds Q and computes S^T = K Q^T, the mask, the row max, the reference
// choice and the weights P = 2^(s - m) (bf16), which it hands to its
// consumer through LDS; the consumer holds O^T and computes O^T += V^T P^T.
// The softmax's vector work of one wave thus runs beside the other wave's
// matrix ops on the same SIMD, while each K or V fragment read from LDS
// still feeds two matrix ops (64 rows), as in the 64-row kernel.
//
// Steps run over 32-key sub-tiles t = 0, 1, ...: at step t the producer
// chooses the reference of t (its rescale factor into alpha slot t % 3),
// computes P(t) (into P buffer t % 2) and S^T(t+1); the consumer applies
// alpha(t-1) to O and adds P(t-1) V(t-1).  A barrier ends each step.
// K and V move through LDS in 64-key stages; at step 2n the producers copy
// K(n+2) and the consumers V(n+1), each waited for at the end of step 2n+2:
// three K and three V stage buffers.
template <int D>
struct WsCfg {
  static constexpr int NP = 4;                    // pairs
  static constexpr int THREADS = 128 * NP;        // 8 waves
  static constexpr int WR = 64;                   // query rows per pair
  static constexpr int BR = NP * WR;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per LDS stage
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = BC * ROWB;
  static constexpr int NKB = 3, NVB = 3;
  static constexpr int KB = 0, VB = NKB * TILE;
  static constexpr int PBUF = 4 * 1024;           // one pair's P of a sub-tile
  static constexpr int PB = VB + NVB * TILE;      // 2 x NP P buffers
  static constexpr int ASLOT = 64 * 8;            // one pair's alpha (2 floats / lane)
  static constexpr int AB = PB + 2 * NP * PBUF;   // 3 x NP alpha slots
  static constexpr int LDS = AB + 3 * NP * ASLOT;
  static constexpr int CHUNKS = D / 8;
  static constexpr int DMA = TILE / 1024 / NP;    // 1 KiB copies per wave per stage
  static constexpr int NC = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int VPF = 3;                   // V fragment lead (fragments)
};
static_assert(W64Cfg<128>::DMA == WsCfg<128>::DMA && W64Cfg<64>::DMA == WsCfg<64>::DMA,
              "copy_stage is shared with the 64-row kernel");

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ s16x8 lds_read_b128_asm(unsigned addr_lds) {
  s16x8 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr_lds));
  return r;
}
__device__ __forceinline__ f32x2 lds_read_b64_asm(unsigned addr_lds) {
  f32x2 r;
  asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(addr_lds));
  return r;
}

template <int D>
struct WsProducer {
  using C = WsCfg<D>;
  bf16x8 qf[2][C::NC];
  float m_ref[2], m_true[2], m_use[2];
  int kaddr[C::NC];
  int voff[C::DMA];
};

template <int D>
struct WsConsumer {
  using C = WsCfg<D>;
  f32x16 oacc[2][C::NDT];
  float l_run[2];          // this lane's half of sum of the bf16 weights
  int vaddr[C::NDT];
  int voff[C::DMA];
};

// Producer step t.  cur = sub-tile t (masked raw scores in s_cur), nxt =
// t+1.  The matrix ops of S^T(nxt) (if has_nxt, from the K rows at kofs)
// carry the vector work of cur: during the first quarter of them the row
// max of cur and the choice of its reference ([RA] §3.2 with the lazy
// reference; rescale factor alpha(t) into al_dst), during the rest the
// weights P(cur) = bf16(2^(s * scale - m)), handed to the consumer at p_dst
// (which sums them into the denominator).  The weights go through three stages
// one step apart (scale and shift, exponential, bf16 and sum), so that no
// instruction waits on the one just before it; every stage's results are
// pinned to their op, as the compiler would otherwise sink the chain.
template <int D>
__device__ __forceinline__ void ws_produce(const AttnArgs& a, char* smem, WsProducer<D>& w,
                                           const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                           const Sub& nxt, bool has_nxt, int kofs, char* p_dst,
                                           char* al_dst, int wq_lo, int lane, int col,
                                           int half) {
  using C = WsCfg<D>;
  constexpr int NSTEP = 2 * C::NC;    // matrix ops (k-step c, block cb)
  constexpr int NMAX = NSTEP / 4;     // ops carrying the row max
  constexpr int NT = 18;              // weight pipeline times (16 pairs + 2)
  const float c_scale = a.scale_log2;
  bf16x8 pb[2][2];
  float tq[16][2], eq[16][2];
  float mq[2][2] = {{-INFINITY, -INFINITY}, {-INFINITY, -INFINITY}};
  // row max: 32 scores of this lane, 32 / NMAX per op, two chains per block
  auto max_part = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    static_for<0, 16 / NMAX>([&](auto yc) {
      constexpr int x = (i * 16 / NMAX + decltype(yc)::value) * 2;  // score index, even
      constexpr int mb = x >> 4, q = x & 15;
      mq[mb][(q >> 1) & 1] = vmax3(mq[mb][(q >> 1) & 1], s_cur[mb][q], s_cur[mb][q + 1]);
    });
  };
  auto decide_cur = [&]() {
    float alpha[2] = {1.0f, 1.0f}, mx[2];
    bool need[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      mx[cb] = pair_max(fmaxf(mq[cb][0], mq[cb][1])) * c_scale;
      w.m_true[cb] = fmaxf(w.m_true[cb], mx[cb]);
      need[cb] = mx[cb] > w.m_ref[cb] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need[0] || need[1])) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        alpha[cb] = need[cb] ? fast_exp2(w.m_ref[cb] - mx[cb]) : 1.0f;
        w.m_ref[cb] = need[cb] ? mx[cb] : w.m_ref[cb];
      }
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) w.m_use[cb] = w.m_ref[cb] == -INFINITY ? 0.0f : w.m_ref[cb];
    *(f32x2*)(al_dst + lane * 8) = f32x2{alpha[0], alpha[1]};
  };
  // weight pipeline time k: bf16 of pair k-2, exponential of pair k-1,
  // scale and shift of pair k (pair x: block x / 8, registers 2 (x % 8), +1)
  auto w_time = [&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k >= 2 && k - 2 < 16) {
      constexpr int x = k - 2, eb = x >> 3, v = 2 * (x & 7);
      pb[eb][v >> 3][v & 7] = (__bf16)eq[x][0];
      pb[eb][v >> 3][(v & 7) + 1] = (__bf16)eq[x][1];
      asm volatile("" ::"v"(pb[eb][v >> 3]));
      // a complete fragment (cb, G) goes to the consumer right away, at
      // p_dst + (2 cb + G) KiB + 16 lane, the layout it reads back
      if constexpr ((x & 3) == 3)
        *(bf16x8*)(p_dst + (2 * eb + (v >> 3)) * 1024 + lane * 16) = pb[eb][v >> 3];
    }
    if constexpr (k >= 1 && k - 1 < 16) {
      constexpr int x = k - 1;
      eq[x][0] = fast_exp2(tq[x][0]);
      eq[x][1] = fast_exp2(tq[x][1]);
      asm volatile("" ::"v"(eq[x][0]), "v"(eq[x][1]));
    }
    if constexpr (k < 16) {
      constexpr int x = k, eb = x >> 3, v = 2 * (x & 7);
      tq[x][0] = fmaf(s_cur[eb][v], c_scale, -w.m_use[eb]);
      tq[x][1] = fmaf(s_cur[eb][v + 1], c_scale, -w.m_use[eb]);
      asm volatile("" ::"v"(tq[x][0]), "v"(tq[x][1]));
    }
  };
  // the pipeline times carried by op i (i >= NMAX)
  auto w_part = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int E = NSTEP - NMAX;
    static_for<(i - NMAX) * NT / E, (i - NMAX + 1) * NT / E>([&](auto kc) { w_time(kc); });
  };
  if (has_nxt) {
    constexpr int PF = 3;
    bf16x8 kf[PF + 1];
    auto kread = [&](int c) -> bf16x8 { return *(const bf16x8*)(smem + kofs + w.kaddr[c]); };
#pragma unroll
    for (int c = 0; c < PF; ++c) kf[c] = kread(c);
    static_for<0, NSTEP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int c = i >> 1, cb = i & 1;
      if constexpr (cb == 0 && c + PF < C::NC) kf[(c + PF) % (PF + 1)] = kread(c + PF);
      s_nxt[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c % (PF + 1)], w.qf[cb][c],
                                                          c == 0 ? f32x16{} : s_nxt[cb], 0, 0, 0);
      if constexpr (i < NMAX) max_part(ic);
      if constexpr (i == NMAX - 1) decide_cur();
      if constexpr (i >= NMAX) w_part(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    static_for<0, NMAX>([&](auto ic) { max_part(ic); });
    decide_cur();
    static_for<0, NT>([&](auto kc) { w_time(kc); });
  }
  if (has_nxt && nxt.mask) {
    mask_sub(s_nxt[0], nxt, a.causal, wq_lo, 0, col, half);
    mask_sub(s_nxt[1], nxt, a.causal, wq_lo, 1, col, half);
  }
}

// Consumer step: O^T *= alpha (when any row's reference moved), then
// O^T += V^T P^T with P from the LDS buffer at p_src and V rows at vofs.
template <int D>
__device__ __forceinline__ void ws_consume(WsConsumer<D>& w, unsigned vofs, unsigned p_src,
                                           unsigned al_src, int lane) {
  using C = WsCfg<D>;
  constexpr int NF = 2 * C::NDT;
  constexpr int NJ = 2 * NF;
  constexpr int PF = C::VPF;
  const f32x2 al = lds_read_b64_asm(al_src + lane * 8);
  s16x8 pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = lds_read_b128_asm(p_src + i * 1024 + lane * 16);
  s16x8 vr[PF + 1];
  auto vread = [&](auto fc) {
    constexpr int f = decltype(fc)::value;
    constexpr int off = (f / C::NDT) * 16 * C::ROWB;
    const unsigned base = vofs + w.vaddr[f % C::NDT];
    const s16x4 lo = lds_read_tr16<off>(base);
    const s16x4 hi = lds_read_tr16<off + 8 * C::ROWB>(base);
    vr[f % (PF + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  static_for<0, PF>([&](auto fc) { vread(fc); });
  f32x2 alc = al;
  claim_lds<4 + 2 * PF>(alc);
  if (__builtin_amdgcn_ballot_w64(alc[0] != 1.0f || alc[1] != 1.0f)) {
    w.l_run[0] *= alc[0];
    w.l_run[1] *= alc[1];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        w.oacc[0][i][v] *= alc[0];
        w.oacc[1][i][v] *= alc[1];
      }
  }
  claim_lds<3 + 2 * PF>(pr[0]);
  claim_lds<2 + 2 * PF>(pr[1]);
  claim_lds<1 + 2 * PF>(pr[2]);
  claim_lds<2 * PF>(pr[3]);
  bf16x8 pb[2][2];
  __builtin_memcpy(&pb[0][0], &pr[0], 16);
  __builtin_memcpy(&pb[0][1], &pr[1], 16);
  __builtin_memcpy(&pb[1][0], &pr[2], 16);
  __builtin_memcpy(&pb[1][1], &pr[3], 16);
  float lp[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  static_for<0, NJ>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int f = j / 2, cb = j % 2;
    // the denominator of P: 16 / NJ bf16 pairs per op (pair x: block x / 8,
    // fragment (x / 4) % 2, elements 2 (x % 4), +1)
    static_for<j * 16 / NJ, (j + 1) * 16 / NJ>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      constexpr int eb = x >> 3, G2 = (x >> 2) & 1, e = 2 * (x & 3);
      const bf16x2 pq = {pb[eb][G2][e], pb[eb][G2][e + 1]};
      lp[eb][x & 1] = __builtin_amdgcn_fdot2_f32_bf16(pq, kOnes2, lp[eb][x & 1], false);
    });
    if constexpr (cb == 0) {
      if constexpr (f + PF < NF) vread(std::integral_constant<int, f + PF>{});
      constexpr int later = 2 * ((f + PF < NF ? f + PF : NF - 1) - f);
      claim_lds<later>(vr[f % (PF + 1)]);
    }
    bf16x8 vf;
    __builtin_memcpy(&vf, &vr[f % (PF + 1)], 16);
    constexpr int G = f / C::NDT, dt = f % C::NDT;
    w.oacc[cb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[cb][G], w.oacc[cb][dt],
                                                             0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  });
  w.l_run[0] += lp[0][0] + lp[0][1];
  w.l_run[1] += lp[1][0] + lp[1][1];
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16_ws(const AttnArgs a) {
  using C = WsCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const bool producer = wave < C::NP;
  const int pair = wave & (C::NP - 1);

  int b, h, qt;
  tile_coords(a, b, h, qt);
  const int row0 = qt * C::BR;
  const int rows_here = min(C::BR, a.Sq - row0);
  const long long q_hi = qpos(a, row0 + rows_here - 1);
  const int wrow0 = row0 + pair * C::WR;
  const int wrows = min(C::WR, a.Sq - wrow0);
  const bool wave_live = wrows > 0;
  const int wq_lo = (int)qpos(a, wrow0);
  const int wq_hi = wq_lo + wrows - 1;
  const int valid_len = a.valid_len > 0x7fffffffLL ? 0x7fffffff : (int)a.valid_len;
  const bool causal = a.causal != 0;
  const long long HD = (long long)a.H * D;
  const int D2 = D * 2;
  const int HD2 = a.Hkv * D2;
  const int hk = h / (a.H / a.Hkv);  // K/V head of this query head
  const unsigned smem_lds = (unsigned)(size_t)(lds_void_ptr)smem;
  // copy slots: producers copy K stages, consumers V stages
  int voff[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int p = (pair * C::DMA + i) * 64 + lane;
    const int r = p / C::CHUNKS, pc = p % C::CHUNKS;
    voff[i] = r * HD2 + (producer ? swz_k<D>(r, pc) : swz_v<D>(r, pc)) * 16;
  }
  const unsigned cdst0 = smem_lds + (producer ? C::KB : C::VB) + pair * C::DMA * 1024;
  char* const p_base = smem + C::PB + pair * C::PBUF;
  char* const a_base = smem + C::AB + pair * C::ASLOT;

  Stage c0 = stage_enter(a, 0, q_hi, b, hk, D2, HD2);    // stage n
  Stage c1 = stage_next(a, c0, q_hi, b, hk, D2, HD2);    // n + 1
  Stage c2 = stage_next(a, c1, q_hi, b, hk, D2, HD2);    // n + 2
  // prologue copies: K(0), K(1) by the producers, V(0) by the consumers
  if (producer) {
    if (c0.blk < a.nblk) copy_stage<D>(c0.k, c0.rows, HD2, voff, cdst0);
    if (c1.blk < a.nblk) copy_stage<D>(c1.k, c1.rows, HD2, voff, cdst0 + C::TILE);
  } else {
    if (c0.blk < a.nblk) copy_stage<D>(c0.v, c0.rows, HD2, voff, cdst0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (producer) {
    WsProducer<D> w;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = wrow0 + 32 * cb + col;
      const __bf16* qp = (const __bf16*)a.q + ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
        w.qf[cb][c] = r < a.Sq ? *(const bf16x8*)(qp + 16 * c + 8 * half) : bf16x8{};
      w.m_ref[cb] = -INFINITY;
      w.m_true[cb] = -INFINITY;
      w.m_use[cb] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < C::NC; ++c) w.kaddr[c] = col * C::ROWB + swz_k<D>(col, 2 * c + half) * 16;
    f32x16 sA[2], sB[2];
    if (c0.blk < a.nblk) {  // S^T of sub-tile 0, its reference
      const Sub s0 = sub_info(c0, 0, causal, valid_len, wq_lo, wq_hi, wave_live);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) sA[cb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        const bf16x8 kf = *(const bf16x8*)(smem + C::KB + w.kaddr[c]);
        sA[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, w.qf[0][c], sA[0], 0, 0, 0);
        sA[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, w.qf[1][c], sA[1], 0, 0, 0);
      }
      if (s0.mask) {
        mask_sub(sA[0], s0, causal, wq_lo, 0, col, half);
        mask_sub(sA[1], s0, causal, wq_lo, 1, col, half);
      }
    }
    int kb0 = 0;  // K buffer of stage n
    for (int n = 0;; ++n) {
      // even step 2n: P(2n), S(2n+1); copy K(n+2)
      const bool live = c0.blk < a.nblk;
      const bool ck = c2.blk < a.nblk;
      if (ck) copy_stage<D>(c2.k, c2.rows, HD2, voff, cdst0 + ((kb0 + 2) % 3) * C::TILE);
      if (live) {
        const Sub s01 = sub_info(c0, 1, causal, valid_len, wq_lo, wq_hi, wave_live);
        ws_produce<D>(a, smem, w, sA, sB, s01, true, C::KB + kb0 * C::TILE + 32 * C::ROWB,
                      p_base, a_base + ((2 * n) % 3) * C::NP * C::ASLOT, wq_lo, lane, col, half);
      }
      if (ck) wait_vmcnt<C::DMA>();
      else wait_vmcnt<0>();
      pipeline_barrier();
      if (!live) break;
      // odd step 2n+1: P(2n+1), S(2n+2)
      {
        const bool has = c1.blk < a.nblk;
        const Sub s10 = sub_info(c1, 0, causal, valid_len, wq_lo, wq_hi, wave_live);
        ws_produce<D>(a, smem, w, sB, sA, s10, has, C::KB + ((kb0 + 1) % 3) * C::TILE,
                      p_base + C::NP * C::PBUF, a_base + ((2 * n + 1) % 3) * C::NP * C::ASLOT,
                      wq_lo, lane, col, half);
      }
      pipeline_barrier();
      c0 = c1;
      c1 = c2;
      c2 = stage_next(a, c2, q_hi, b, hk, D2, HD2);
      kb0 = kb0 == 2 ? 0 : kb0 + 1;
    }
    // hand the reference and the exact max of every row to the consumer
    if (half == 0) {
      *(f32x2*)(a_base + col * 8) = f32x2{w.m_ref[0], w.m_ref[1]};
      *(f32x2*)(a_base + 256 + col * 8) = f32x2{w.m_true[0], w.m_true[1]};
    }
    __syncthreads();
  } else {
    WsConsumer<D> w;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int i = 0; i < C::NDT; ++i) w.oacc[cb][i] = f32x16{};
      w.l_run[cb] = 0.0f;
    }
    {
      const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
      const int kl = 4 * half + e;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
        w.vaddr[dt] = kl * C::ROWB + swz_v<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
      }
    }
    const unsigned p0 = (unsigned)(size_t)(lds_void_ptr)p_base;
    const unsigned al0 = (unsigned)(size_t)(lds_void_ptr)a_base;
    int vbp = 2;  // V buffer of stage n - 1
    for (int n = 0;; ++n) {
      // even step 2n: P(2n-1) V(2n-1); copy V(n+1)
      const bool live = c0.blk < a.nblk;
      const bool cv = c1.blk < a.nblk;
      const int vb0 = vbp == 2 ? 0 : vbp + 1;
      if (cv) copy_stage<D>(c1.v, c1.rows, HD2, voff, cdst0 + ((vb0 + 1) % 3) * C::TILE);
      if (n > 0)
        ws_consume<D>(w, smem_lds + C::VB + vbp * C::TILE + 32 * C::ROWB,
                      p0 + C::NP * C::PBUF, al0 + ((2 * n - 1) % 3) * C::NP * C::ASLOT, lane);
      if (cv) wait_vmcnt<C::DMA>();
      else wait_vmcnt<0>();
      pipeline_barrier();
      if (!live) break;
      // odd step 2n+1: P(2n) V(2n)
      ws_consume<D>(w, smem_lds + C::VB + vb0 * C::TILE, p0,
                    al0 + ((2 * n) % 3) * C::NP * C::ASLOT, lane);
      pipeline_barrier();
      c0 = c1;
      c1 = c2;
      c2 = stage_next(a, c2, q_hi, b, hk, D2, HD2);
      vbp = vb0;
    }
    __syncthreads();  // the producer's reference and max
    const f32x2 m_ref = *(const f32x2*)(a_base + col * 8);
    const f32x2 m_true = *(const f32x2*)(a_base + 256 + col * 8);
    // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float l_tot = pair_sum(w.l_run[cb]);
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const int r = wrow0 + 32 * cb + col;
      if (half == 0 && r < a.Sq) {
        const long long so = ((long long)b * a.Sq + r) * a.H + h;
        const bool seen = l_tot > 0.0f;
        if (a.lse) a.lse[so] = seen ? (m_ref[cb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
        if (a.m_out) a.m_out[so] = seen ? m_true[cb] * kLn2 : -INFINITY;
        if (a.l_out) a.l_out[so] = seen ? l_tot * fast_exp2(m_ref[cb] - m_true[cb]) : 0.0f;
      }
      if (r >= a.Sq) continue;
      const long long ro = ((long long)b * a.Sq + r) * HD + (long long)h * D;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * half;
          const float x0 = w.oacc[cb][dt][4 * g + 0] * inv, x1 = w.oacc[cb][dt][4 * g + 1] * inv;
          const float x2 = w.oacc[cb][dt][4 * g + 2] * inv, x3 = w.oacc[cb][dt][4 * g + 3] * inv;
          if (a.o_fp32) {
            *(float4*)((float*)a.o + ro + d) = float4{x0, x1, x2, x3};
          } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 y;
            y[0] = (__bf16)x0; y[1] = (__bf16)x1; y[2] = (__bf16)x2; y[3] = (__bf16)x3;
            *(bf16x4*)((__bf16*)a.o + ro + d) = y;
          }
        }
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
  const long long q_hi = qpos(a, row0 + rows_here - 1);
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = qpos(a, wrow0);
  const long long wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;
  const long long HDkv = (long long)a.Hkv * D;
  const int hk = h / (a.H / a.Hkv);  // K/V head of this query head

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
    const float* kp = (const float*)kb.k + ((long long)b * a.kv_rows_b + kt0) * HDkv + (long long)hk * D;
    const float* vp = (const float*)kb.v + ((long long)b * a.kv_rows_b + kt0) * HDkv + (long long)hk * D;
    const int rows = min(BC, kb.len - kt0);
#pragma unroll
    for (int u = 0; u < C::UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int r = unit / (D / 4), c = unit % (D / 4);
      kreg[u] = r < rows ? *(const float4*)(kp + r * HDkv + 4 * c) : float4{0, 0, 0, 0};
      vreg[u] = r < rows ? *(const float4*)(vp + r * HDkv + 4 * c) : float4{0, 0, 0, 0};
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
// Kernel choice for bf16 (RA_OPT_ATTN_KERNEL): 4 or 8 waves of 32 rows
// (two waves per SIMD), 4 waves of 64 rows (one wave per SIMD), 4
// producer / consumer pairs of 64 rows (two waves per SIMD), or the
// ping-pong form of 8 waves of 32 rows.
enum Bf16Kernel { K_BR128, K_BR256, K_W64, K_WS, K_PP };

// The 64-row kernel keeps positions in 32 bits: usable when every query
// and key position (plus a tile of slack) stays below 2^31.
bool positions_fit_32(const AttnArgs& a) {
  const long long lim = 0x7fffffffLL - 256;
  if (qpos(a, a.Sq - 1) + 1 > lim) return false;
  for (int i = 0; i < a.nblk; ++i)
    if (a.blk[i].k_pos0 + a.blk[i].len > lim) return false;
  return true;
}

Bf16Kernel bf16_kernel(const AttnArgs& a) {
  const int mode = ra::option(RA_OPT_ATTN_KERNEL);
  if (mode == RA_KERNEL_BR128) return K_BR128;
  if (mode == RA_KERNEL_BR256) return K_BR256;
  if (mode == RA_KERNEL_W64) return positions_fit_32(a) ? K_W64 : K_BR128;
  if (mode == RA_KERNEL_WS) return positions_fit_32(a) ? K_WS : K_BR128;
  if (mode == RA_KERNEL_PP) return K_PP;
  return K_BR128;
}

template <int NW>
void launch_bf16(const AttnArgs& a, int D, dim3 grid, hipStream_t stream) {
  if (D == 128) hipLaunchKernelGGL((ring_attn_bf16<128, NW>), grid, dim3(64 * NW), 0, stream, a);
  else hipLaunchKernelGGL((ring_attn_bf16<64, NW>), grid, dim3(64 * NW), 0, stream, a);
}

ra_status launch(AttnArgs& a, int D, ra_dtype dt, hipStream_t stream, const char* name) {
  // a split ring runs on the 128-row kernel (its slots hold 128 rows)
  const bool split = a.nsplit > 1;
  const Bf16Kernel kk = dt != RA_BF16 || split ? K_BR128 : bf16_kernel(a);
  const int br = dt != RA_BF16 ? kBR : kk == K_BR128 ? 128 : 256;
  a.n_qtiles = (a.Sq + br - 1) / br;
  const long long n_wg = (long long)a.B * a.H * a.n_qtiles * (split ? a.nsplit : 1);
  if (n_wg == 0) return RA_OK;
  if (n_wg > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: too many query tiles", name);
  const dim3 grid((unsigned)n_wg);
  if (dt == RA_BF16) {
    if (kk == K_W64) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bf16_w64<128>, grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(ring_attn_bf16_w64<64>, grid, dim3(256), 0, stream, a);
    } else if (kk == K_WS) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bf16_ws<128>, grid, dim3(512), 0, stream, a);
      else hipLaunchKernelGGL(ring_attn_bf16_ws<64>, grid, dim3(512), 0, stream, a);
    } else if (kk == K_PP) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bf16_pp<128>, grid, dim3(512), 0, stream, a);
      else hipLaunchKernelGGL(ring_attn_bf16_pp<64>, grid, dim3(512), 0, stream, a);
    } else if (kk == K_BR256) {
      launch_bf16<8>(a, D, grid, stream);
    } else if (split) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bf16_split<128>, grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(ring_attn_bf16_split<64>, grid, dim3(256), 0, stream, a);
    } else {
      launch_bf16<4>(a, D, grid, stream);
    }
  } else {
    if (D == 128) hipLaunchKernelGGL(ring_attn_f32<128>, grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(ring_attn_f32<64>, grid, dim3(kThreads), 0, stream, a);
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
  a.q_pos1 = q_pos0 + Sq;
  a.q_split = Sq;
  a.kv_rows_b = Sk;
  a.Hkv = H;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
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

namespace {
// Split of the ring set up in `a` (blocks, positions, causal, valid_len):
// every 128-row query tile's visited-tile sequence in ns runs.  ns = 0
// chooses: as many runs as keep the B*H*n_qtiles*ns workgroups within the
// chip's slots (one round, two per compute unit), each run at least
// kSplitMinRun tiles of the longest sequence; 1 (no split) when the single
// pass already fills the slots.  Returns the run count (1: no split) and, in
// ws, the workspace floats (partial o and lse slots) it needs.
constexpr int kSplitMinRun = 8;  // tiles: 512 keys per workgroup at least

int split_plan(const AttnArgs& a, int D, int ns, long long& ws) {
  ws = 0;
  const int n_qt = (a.Sq + 127) / 128;
  const long long base = (long long)a.B * a.H * n_qt;
  if (base <= 0) return 1;
  if (ns <= 0) {
    if (base >= ra::kWorkgroupSlots) return 1;
    int max_t = 0;
    for (int qt = 0; qt < n_qt; ++qt) {
      const long long q_hi = qpos(a, (qt + 1) * 128 < a.Sq ? (qt + 1) * 128 - 1 : a.Sq - 1);
      int t = 0;
      for (int bi = 0; bi < a.nblk; ++bi) t += tiles_of<64>(a, bi, q_hi);
      if (t > max_t) max_t = t;
    }
    ns = (int)(ra::kWorkgroupSlots / base);
    if (ns > max_t / kSplitMinRun) ns = max_t / kSplitMinRun;
  }
  if (ns <= 1) return 1;
  ws = base * ns * 128 * (long long)(D + 1);
  return ns;
}

// The whole ring of one rank (shared by the MHA and GQA entry points).
ra_status ring_fwd(const char* name, const void* q_r, const void* const* k_blocks,
                   const void* const* v_blocks, int B, int Sb, int H, int Hkv, int D, int P,
                   int rank, ra_dtype dt, float scale, int causal, long long valid_len, void* o,
                   float* lse_opt, void* stream, int nsplit = 1, float* ws = nullptr,
                   long long ws_floats = 0) {
  ra::clear_error();
  ra_status st = check_common(name, B, Sb, H, D, dt);
  if (st != RA_OK) return st;
  if (Hkv <= 0 || H % Hkv != 0)
    return ra::fail(RA_ERR_SHAPE, "%s: %d query heads are not a multiple of %d K/V heads",
                    name, H, Hkv);
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
  a.q_pos1 = a.q_pos0 + Sb;
  a.q_split = Sb;
  a.kv_rows_b = Sb;
  a.Hkv = Hkv;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sb;
  a.H = H;
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
  if (nsplit > 1 && dt == RA_BF16) {
    long long need = 0;
    const int ns = split_plan(a, D, nsplit, need);
    if (ns > 1) {
      if (!ws) return ra::fail(RA_ERR_NULL, "%s: NULL split workspace", name);
      if (ws_floats < need)
        return ra::fail(RA_ERR_SHAPE, "%s: split workspace of %lld floats, %lld needed", name,
                        ws_floats, need);
      if (!aligned16(ws)) return ra::fail(RA_ERR_SHAPE, "%s: workspace not 16-byte aligned", name);
      const long long slots = (long long)B * H * ((Sb + 127) / 128) * ns;
      ra::SplitMergeArgs m{};
      m.o_part = ws;
      m.lse_part = ws + slots * 128 * D;
      m.o = o;
      m.lse = lse_opt;
      m.B = B;
      m.Sq = Sb;
      m.H = H;
      m.D = D;
      m.nsplit = ns;
      m.out_bf16 = 1;
      a.nsplit = ns;
      a.o = ws;
      a.lse = ws + slots * 128 * D;
      a.o_fp32 = 1;
      st = launch(a, D, dt, (hipStream_t)stream, name);
      if (st != RA_OK) return st;
      return ra::merge_split(name, m, stream);
    }
  }
  return launch(a, D, dt, (hipStream_t)stream, name);
}
}  // namespace

extern "C" ra_status ra_ring_attn_fwd_varlen(const void* q_r, const void* const* k_blocks,
                                             const void* const* v_blocks, int Sb, int H, int D,
                                             int P, int rank, ra_dtype dt, float scale,
                                             int causal, const long long* cu_seqlens,
                                             int n_seqs, void* o, float* lse_opt,
                                             void* stream) {
  static const char* name = "ra_ring_attn_fwd_varlen";
  ra::clear_error();
  ra_status st = check_common(name, 1, Sb, H, D, dt);
  if (st != RA_OK) return st;
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (P > RA_MAX_P)
    return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P=%d", name, P, RA_MAX_P);
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
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
  if (!q_r || !o || !k_blocks || !v_blocks)
    return ra::fail(RA_ERR_NULL, "%s: NULL q/o/block table", name);
  if (!aligned16(q_r) || !aligned16(o))
    return ra::fail(RA_ERR_SHAPE, "%s: q and o must be 16-byte aligned", name);
  const size_t row_bytes = (size_t)H * D * (dt == RA_BF16 ? 2 : 4);
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  const long long q0 = (long long)rank * Sb, q1 = q0 + Sb;
  int src[RA_MAX_P], cls[RA_MAX_P];
  st = ra_ring_schedule(P, rank, Sb, causal, S, src, cls);
  if (st != RA_OK) return st;
  // one launch per sample that meets the rank's rows: its rows of the share
  // against the parts of the visited blocks that lie inside the sample, in
  // ring order (a packed sequence never attends across samples)
  for (int i = 0; i < n_seqs; ++i) {
    const long long s0 = cu_seqlens[i], s1 = cu_seqlens[i + 1];
    const long long r0 = s0 > q0 ? s0 : q0, r1 = s1 < q1 ? s1 : q1;
    if (r1 <= r0) continue;
    AttnArgs a{};
    a.q = (const char*)q_r + (size_t)(r0 - q0) * row_bytes;
    a.o = (char*)o + (size_t)(r0 - q0) * row_bytes;
    a.lse = lse_opt ? lse_opt + (r0 - q0) * H : nullptr;
    a.q_pos0 = r0;
    a.q_pos1 = r1;
    a.q_split = (int)(r1 - r0);
    a.kv_rows_b = Sb;  // B = 1: never used for a stride
    a.Hkv = H;
    a.valid_len = s1;  // keys past the sample's end are not real for it
    a.B = 1;
    a.Sq = (int)(r1 - r0);
    a.H = H;
    a.causal = causal != 0;
    a.o_fp32 = dt == RA_FP32;
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    a.nblk = 0;
    for (int t = 0; t < P; ++t) {
      if (cls[t] == RA_SKIP) continue;
      const int j = src[t];
      const long long b0 = (long long)j * Sb, b1 = b0 + Sb;
      const long long k0 = b0 > s0 ? b0 : s0, k1 = b1 < s1 ? b1 : s1;
      if (k1 <= k0) continue;
      const int c = ra::block_class(r0, r1, k0, k1, causal != 0, s1);
      if (c == RA_SKIP) continue;
      if (!k_blocks[j] || !v_blocks[j])
        return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited block %d", name, j);
      if (!aligned16(k_blocks[j]) || !aligned16(v_blocks[j]))
        return ra::fail(RA_ERR_SHAPE, "%s: block %d not 16-byte aligned", name, j);
      const size_t off = (size_t)(k0 - b0) * row_bytes;
      a.blk[a.nblk++] = KVBlock{(const char*)k_blocks[j] + off, (const char*)v_blocks[j] + off,
                                k0, (int)(k1 - k0), c};
    }
    st = launch(a, D, dt, (hipStream_t)stream, name);
    if (st != RA_OK) return st;
  }
  return RA_OK;
}

extern "C" ra_status ra_ring_attn_fwd(const void* q_r, const void* const* k_blocks,
                                      const void* const* v_blocks, int B, int Sb,
                                      int H, int D, int P, int rank, ra_dtype dt,
                                      float scale, int causal, long long valid_len,
                                      void* o, float* lse_opt, void* stream) {
  return ring_fwd("ra_ring_attn_fwd", q_r, k_blocks, v_blocks, B, Sb, H, H, D, P, rank, dt,
                  scale, causal, valid_len, o, lse_opt, stream);
}

extern "C" ra_status ra_ring_attn_fwd_gqa(const void* q_r, const void* const* k_blocks,
                                          const void* const* v_blocks, int B, int Sb, int H,
                                          int H_kv, int D, int P, int rank, ra_dtype dt,
                                          float scale, int causal, long long valid_len,
                                          void* o, float* lse_opt, void* stream) {
  return ring_fwd("ra_ring_attn_fwd_gqa", q_r, k_blocks, v_blocks, B, Sb, H, H_kv, D, P, rank,
                  dt, scale, causal, valid_len, o, lse_opt, stream);
}

extern "C" ra_status ra_ring_attn_fwd_split(const void* q_r, const void* const* k_blocks,
                                            const void* const* v_blocks, int B, int Sb, int H,
                                            int Hkv, int D, int P, int rank, ra_dtype dt,
                                            float scale, int causal, long long valid_len,
                                            int nsplit, float* ws, long long ws_floats, void* o,
                                            float* lse_opt, void* stream) {
  if (nsplit < 1) {
    ra::clear_error();
    return ra::fail(RA_ERR_RANGE, "ra_ring_attn_fwd_split: nsplit must be >= 1 (got %d)",
                    nsplit);
  }
  return ring_fwd("ra_ring_attn_fwd_split", q_r, k_blocks, v_blocks, B, Sb, H, Hkv, D, P, rank,
                  dt, scale, causal, valid_len, o, lse_opt, stream, nsplit, ws, ws_floats);
}

extern "C" int ra_ring_split_plan(int B, int Sb, int H, int D, int P, int rank, int causal,
                                  long long valid_len, int nsplit, long long* ws_floats) {
  static const char* name = "ra_ring_split_plan";
  ra::clear_error();
  if (ws_floats) *ws_floats = 0;
  if (B < 0 || Sb < 0 || H < 0 || (D != 64 && D != 128) || P <= 0 || P > RA_MAX_P) {
    ra::fail(RA_ERR_SHAPE, "%s: bad sizes (B=%d Sb=%d H=%d D=%d P=%d)", name, B, Sb, H, D, P);
    return -1;
  }
  if (rank < 0 || rank >= P) {
    ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
    return -1;
  }
  if (nsplit < 0) {
    ra::fail(RA_ERR_RANGE, "%s: nsplit must be >= 0", name);
    return -1;
  }
  const long long S = (long long)P * Sb;
  if (valid_len < 0 || valid_len > S) valid_len = S;
  AttnArgs a{};
  a.q_pos0 = (long long)rank * Sb;
  a.q_pos1 = a.q_pos0 + Sb;
  a.q_split = Sb;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sb;
  a.H = H;
  a.causal = causal != 0;
  int src[RA_MAX_P], cls[RA_MAX_P];
  if (ra_ring_schedule(P, rank, Sb, causal, valid_len, src, cls) != RA_OK) return -1;
  for (int t = 0; t < P; ++t)
    if (cls[t] != RA_SKIP)
      a.blk[a.nblk++] = KVBlock{nullptr, nullptr, (long long)src[t] * Sb, Sb, cls[t]};
  long long need = 0;
  const int ns = split_plan(a, D, nsplit, need);
  if (ws_floats) *ws_floats = need;
  return ns;
}

extern "C" ra_status ra_zigzag_attn_fwd(const void* q_r, const void* const* k_shares,
                                        const void* const* v_shares, int B, int Sr, int H,
                                        int D, int P, int rank, ra_dtype dt, float scale,
                                        int causal, long long valid_len, void* o,
                                        float* lse_opt, void* stream) {
  static const char* name = "ra_zigzag_attn_fwd";
  ra::clear_error();
  ra_status st = check_common(name, B, Sr, H, D, dt);
  if (st != RA_OK) return st;
  if (P <= 0) return ra::fail(RA_ERR_SHAPE, "%s: P must be positive (got %d)", name, P);
  if (2 * P > RA_MAX_P)
    return ra::fail(RA_ERR_RANGE, "%s: P=%d exceeds RA_MAX_P/2=%d", name, P, RA_MAX_P / 2);
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "%s: rank %d outside [0, %d)", name, rank, P);
  if (Sr % 128 != 0)
    return ra::fail(RA_ERR_SHAPE, "%s: rows per rank (%d) must be two chunks of a multiple "
                    "of 64 rows; pad the sequence to ra_zigzag_padded_len(S, P)", name, Sr);
  const long long n_out = (long long)B * Sr * H;
  if (n_out == 0) return RA_OK;
  if (!q_r || !o || !k_shares || !v_shares)
    return ra::fail(RA_ERR_NULL, "%s: NULL q/o/share table", name);
  if (!aligned16(q_r) || !aligned16(o))
    return ra::fail(RA_ERR_SHAPE, "%s: q and o must be 16-byte aligned", name);
  const int c = Sr / 2;  // chunk length
  const long long S = (long long)P * Sr;
  if (valid_len < 0 || valid_len > S) valid_len = S;
  AttnArgs a{};
  a.q = q_r;
  a.o = o;
  a.lse = lse_opt;
  // the share is chunk rank (rows [0, c)) then chunk 2P-1-rank (rows [c, 2c))
  a.q_pos0 = (long long)rank * c;
  a.q_pos1 = (long long)(2 * P - 1 - rank) * c;
  a.q_split = c;
  a.kv_rows_b = Sr;
  a.Hkv = H;
  a.valid_len = valid_len;
  a.B = B;
  a.Sq = Sr;
  a.H = H;
  a.causal = causal != 0;
  a.o_fp32 = dt == RA_FP32;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  // round t visits the share of rank (rank - t) mod P, as in the plain ring;
  // each share is two chunks, classified against the whole query share
  int src[RA_MAX_P], cls[2 * RA_MAX_P];
  st = ra_zigzag_schedule(P, rank, c, causal, valid_len, src, cls);
  if (st != RA_OK) return st;
  a.nblk = 0;
  const size_t row_bytes = (size_t)H * D * (dt == RA_BF16 ? 2 : 4);
  for (int t = 0; t < P; ++t) {
    const int j = src[t];
    for (int half = 0; half < 2; ++half) {
      if (cls[2 * t + half] == RA_SKIP) continue;
      if (!k_shares[j] || !v_shares[j])
        return ra::fail(RA_ERR_NULL, "%s: NULL pointer for visited share %d", name, j);
      if (!aligned16(k_shares[j]) || !aligned16(v_shares[j]))
        return ra::fail(RA_ERR_SHAPE, "%s: share %d not 16-byte aligned", name, j);
      const int chunk = half == 0 ? j : 2 * P - 1 - j;
      const size_t off = (size_t)half * c * row_bytes;
      a.blk[a.nblk++] = KVBlock{(const char*)k_shares[j] + off, (const char*)v_shares[j] + off,
                                (long long)chunk * c, c, cls[2 * t + half]};
    }
  }
  return launch(a, D, dt, (hipStream_t)stream, name);
}
