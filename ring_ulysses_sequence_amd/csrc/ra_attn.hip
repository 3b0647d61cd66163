// Ring-order block attention on CDNA4 (gfx950): the local query shard stays
// on chip while K/V blocks stream through LDS in ring order, merged by the
// online-softmax recurrence ([RA] §3.2-§3.4).
//
// One workgroup = 4 or 8 wavefronts = 128 or 256 query rows of one (batch,
// head); each wave owns 32 rows.  Per K/V tile of 64 keys a wave computes the
// TRANSPOSED score tile S^T = K Q^T on the matrix cores, so that every lane
// holds the scores of one query column: the row max is an in-lane reduction
// plus one cross-half exchange (v_permlane32_swap), not a 32-lane butterfly.
// The bf16 kernels take the row sum on the matrix cores as well (a 0/1
// selector times the P fragments); the fp32 kernel reduces it like the max.
// The probabilities P^T then feed O^T += V^T P^T directly as the B operand;
// the V^T operand is read from row-major V in LDS by transposing reads.
//
// Matrix-core operand layouts used below (64-lane wave, l = lane,
// col = l % 32, half = l / 32):
//   32x32x16 bf16  A[m][k]: lane holds m = col, k = 8*half .. 8*half+7
//                  B[k][n]: lane holds n = col, k = 8*half .. 8*half+7
//                  C[m][n]: lane holds n = col, m = 8*(v/4) + 4*half + v%4,
//                           v = 0..15
//   32x32x2 f32    A: m = col, k = half;  B: n = col, k = half;  C as above.
//   16x16x32 bf16  A[m][k]: lane holds m = l % 16, k = 8*(l/16) .. +7
//                  B[k][n]: lane holds n = l % 16, k = 8*(l/16) .. +7
//                  C[m][n]: lane holds n = l % 16, m = 4*(l/16) + v, v = 0..3
// A contraction index may be permuted freely as long as A and B agree; both
// operands below are built with the same (half, element) -> index map.
//
// K/V tiles are multi-buffered in LDS and copied by the buffer unit straight
// from HBM into LDS (no staging registers): while a tile is consumed, the
// tiles two or three steps ahead -- possibly the first tiles of the next ring round
// -- are in flight, so the stream continues across round boundaries without
// a drain.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <algorithm>
#include <vector>
#include <type_traits>

#include "ra_internal.h"
#include "ra_order.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Everything of one attention problem but its block table.
struct AttnHead {
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
  int rowmax;          // take the row max of every tile (RA_KERNEL_ROWMAX)
  // accumulate mode (acc != 0, never split): o (fp32) and lse hold the
  // running partial of the blocks folded in so far; the epilogue combines
  // this launch's partial with it and writes the result back, or -- with
  // o_final -- writes the combined output in the input dtype to o_final and
  // only lse back
  int acc;
  void* o_final;
  // rotation of the block table for the later query tiles of the lockstep
  // order (ra_order.h), 0 for none: 1 for a ring share whose visited blocks
  // after the first are FULL, 2 for a causal zigzag share (its own two
  // chunks first); the 8-wave kernel then visits their blocks from that
  // table entry on, wrapping around
  int lockstep;
  int nblk;
};
// A problem with room for N visited blocks; AttnArgs (RA_MAX_P) for a whole
// ring, a smaller table where many problems share one launch's arguments.
template <int N>
struct AttnArgsT : AttnHead {
  KVBlock blk[N];
};
using AttnArgs = AttnArgsT<RA_MAX_P>;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2eF = 1.4426950408889634f;

template <class A>
__host__ __device__ __forceinline__ long long qpos(const A& a, int row) {
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
template <int BC, class A>
__host__ __device__ __forceinline__ int tiles_of(const A& a, int b, long long q_hi) {
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

template <class A>
__device__ __forceinline__ void tile_coords_in(const A& a, int id, int& b, int& h,
                                               int& qt) {
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
// Lockstep order (ra_order.h) for the 8-wave ring kernel.  The result is
// the ring's up to the order in which the online softmax folds the blocks in.
template <class A>
__device__ __forceinline__ bool tile_coords_lockstep(const A& a, int id, int n, int& b,
                                                     int& h, int& qt, int& rot) {
  int bh;
  if (!a.lockstep || a.nblk <= 0 ||
      !ra_order::lockstep_coords(id, n, a.n_qtiles, a.B * a.H, a.lockstep % a.nblk, bh, qt,
                                 rot))
    return false;
  h = bh % a.H;
  b = bh / a.H;
  return true;
}
template <class A>
__device__ __forceinline__ void tile_coords(const A& a, int id, int n, int& b, int& h,
                                            int& qt) {
  if ((n & 7) == 0) id = (id & 7) * (n >> 3) + (id >> 3);
  tile_coords_in(a, id, b, h, qt);
}
template <class A>
__device__ __forceinline__ void tile_coords(const A& a, int& b, int& h, int& qt) {
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
// Software pipeline (per wave, step n over the visited tiles; tiles are
// copied LEAD steps ahead, LEAD = 2 with 4 waves, 3 with 8):
//   copy K(n+LEAD) and V(n+LEAD) into buffers that earlier steps released;
//   front: S^T(n+1) = K(n+1) Q^T on the matrix cores, interleaved with the
//          exponentials of the second half (keys 32..63) of tile n;
//   back:  O^T += V(n)^T P(n)^T on the matrix cores, interleaved with the
//          mask and the exponentials of the first half of tile n+1;
//   wait for this wave's copies of K(n+2) and V(n+1) (later ones may stay
//   in flight), barrier.
// Every matrix phase thus carries half a tile of softmax work, so a wave on
// its own keeps the matrix pipe fed, and the second wave of the SIMD fills
// what is left.  4 waves: two K and three V buffers (80 KiB at D = 128, two
// workgroups per CU), buffer indices at run time, the loop unrolled by two
// (the score and P register sets swap roles).  8 waves: four K and four V
// buffers (128 KiB, one workgroup per CU) and the loop unrolled by four, so
// that every buffer index is a constant and the operand reads carry the
// buffer offset as an immediate.  Operand reads run four matrix ops ahead
// of their use.
//
// Reference max ([RA] §3.2 with a moving reference).  P is formed as
// 2^(s - m_ref) against a per-row reference m_ref that u and l share, so
// u / l is the quotient of the recurrence whatever the reference is.  The
// reference is set to a row's exact max on its first tile with a visible
// key; after that the row max is not recomputed per tile.  Instead the sum
// of each tile's weights (computed anyway for l) is checked: while every
// weight stays below 2^20 nothing can overflow, and a tile whose sum
// exceeds that bound or is NaN (a score more than ~20 above the reference,
// or an infinite weight) is redone after moving the reference to that tile's
// max and rescaling u and l.  RA_KERNEL_ROWMAX takes the row max of every
// tile instead and moves the reference lazily (when the max exceeds it by
// more than 8); the same path runs whenever m and l are requested.
template <int D, int NW_>
struct Bf16Cfg {
  static constexpr int NW = NW_;                  // waves per workgroup (4 or 8)
  static constexpr int THREADS = 64 * NW;
  static constexpr int BR = 32 * NW;              // query rows per workgroup
  static constexpr int BC = 64;                   // keys per tile
  static constexpr int ROWB = D * 2;              // bytes per key row in LDS
  static constexpr int TILE = BC * ROWB;          // one K or V tile
  // copies of tile n + LEAD are issued in step n: two K and three V buffers
  // for 4 waves (80 KiB at D = 128, two workgroups per CU), four and four
  // for 8 waves (128 KiB, one workgroup per CU).  The 8-wave loop runs four
  // steps per iteration, so that every buffer index in it is a constant and
  // the operand reads take the buffer offset as an immediate.
  static constexpr int LEAD = NW == 8 ? 3 : 2;
  static constexpr int KBUF = NW == 8 ? 4 : LEAD;
  static constexpr int VBUF = LEAD + 1;
  static constexpr bool FIXED = NW == 8;
  static constexpr int KB = 0;                    // K buffers at KB + p*TILE
  static constexpr int VB = KBUF * TILE;          // V buffers at VB + p*TILE
  static constexpr int LDS = (KBUF + VBUF) * TILE;
  static constexpr int CHUNKS = D / 8;            // 16-byte chunks per row
  static constexpr int DMA = TILE / 1024 / NW;    // 1 KiB copies per wave per tile
  static constexpr int NC = D / 16;               // k-steps of S^T = K Q^T
  static constexpr int NDT = D / 32;              // 32-row d tiles of O^T
  static constexpr int NQK = 2 * NC;              // matrix ops of S^T per tile
  static constexpr int NPV = 4 * NDT;             // matrix ops of O^T per tile
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access
constexpr float kRescaleSlack = 8.0f;   // lazy move of the reference (base-2 units)
constexpr float kTileSumLimit = 1048576.0f;  // 2^20: bound on one half tile's weights
constexpr int kOperandLead = 4;  // LDS operand reads run this many matrix ops ahead

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS operand reads as inline assembly.  The compiler's own LDS reads wait
// for every LDS-DMA copy in flight (it cannot tell which LDS bytes a copy
// writes), which would stall each matrix phase on the copies issued at the
// start of the same step.  These reads are invisible to the compiler's wait
// insertion, so each result is claimed with claim_lds<N> before use; the
// copies they must not overtake are ordered by the explicit waits and
// barriers of the pipeline.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  bf16x8 x;
  __builtin_memcpy(&x, &r, 16);
  return x;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
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

// ---- the visited-tile sequence -------------------------------------------
// A workgroup visits the tiles of every visited block in ring order, each
// block up to the last tile with a key visible to the workgroup's last
// query ([RA] §3.4 applied per tile; tiles wholly in the future or wholly
// padding are never read).  All waves of a workgroup walk the same sequence
// (they share the copies); positions are taken relative to each wave's
// first query so that the per-tile tests are 32-bit scalar arithmetic.
struct SeqCtx {
  long long q_hi;    // the workgroup's last query position
  long long wq_lo;   // this wave's first query position
  long long boff;    // byte offset of (batch b, K/V head) row 0 in a block
  int end_blk, end_t;  // the sequence ends before tile end_t of block end_blk
  int rot;           // visit the table from entry rot on, wrapping around
};

// Table entry of the p-th visited block.
template <class A>
__device__ __forceinline__ int seq_bidx(const A& a, const SeqCtx& x, int p) {
  const int i = p + x.rot;
  return i >= a.nblk ? i - a.nblk : i;
}

// Cursor over the sequence; blk == a.nblk once past its end.  Everything
// here is wave-uniform; the block fields are loaded once per block.
struct Seq {
  int blk, t, n;     // block, tile in it, visited tiles of it
  int len;           // rows of the block
  int rel0;          // block's first key position - wave's first query position
  int lim0;          // real keys of the block, min(len, valid_len - first key)
  const char* kp;    // K row 0 of (b, K/V head) in the block
  const char* vp;    // V row 0
};

// Per-tile facts a step needs about a tile (carried along the pipeline).
struct TDesc {
  int valid;         // the tile exists
  int rel;           // first key position - wave's first query position
  int lim;           // real keys in the tile (1..64)
};

__device__ __forceinline__ long long clampll(long long x, long long lo, long long hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Move s to the first block at or after s.blk with visited tiles (t = 0).
template <class A>
__device__ __forceinline__ void seq_enter(const A& a, const SeqCtx& x, Seq& s) {
  s.t = 0;
  for (; s.blk < a.nblk; ++s.blk) {
    s.n = tiles_of<64>(a, seq_bidx(a, x, s.blk), x.q_hi);
    if (s.n > 0) break;
  }
  if (s.blk >= a.nblk) return;
  const KVBlock& kb = a.blk[seq_bidx(a, x, s.blk)];
  s.len = kb.len;
  s.kp = (const char*)kb.k + x.boff;
  s.vp = (const char*)kb.v + x.boff;
  // clamps keep rel0 + 64 t and lim0 - 64 t inside 32 bits (len <= 2^30)
  s.rel0 = (int)clampll(kb.k_pos0 - x.wq_lo, -(1LL << 30), 1LL << 29);
  const long long lim = a.valid_len - kb.k_pos0;
  s.lim0 = (int)clampll(lim < kb.len ? lim : kb.len, 0, 1LL << 30);
}
template <class A>
__device__ __forceinline__ void seq_clip(const A& a, const SeqCtx& x, Seq& s) {
  if (s.blk > x.end_blk || (s.blk == x.end_blk && s.t >= x.end_t)) s.blk = a.nblk;
}
template <class A>
__device__ __forceinline__ void seq_next(const A& a, const SeqCtx& x, Seq& s) {
  if (s.blk >= a.nblk) return;
  if (++s.t >= s.n) {
    ++s.blk;
    seq_enter(a, x, s);
  }
  seq_clip(a, x, s);
}
// Block and tile of tile number i of the sequence (blk = a.nblk past it).
template <class A>
__device__ __forceinline__ void seq_locate(const A& a, const SeqCtx& x, int i, int& blk,
                                           int& t) {
  for (blk = 0; blk < a.nblk; ++blk) {
    const int n = tiles_of<64>(a, seq_bidx(a, x, blk), x.q_hi);
    if (i < n) break;
    i -= n;
  }
  t = i;
}
template <class A>
__device__ __forceinline__ Seq seq_first(const A& a, const SeqCtx& x, int lo) {
  Seq s{};
  seq_locate(a, x, lo, s.blk, s.t);
  const int t = s.t;
  if (s.blk < a.nblk) {
    seq_enter(a, x, s);  // the located block has visited tiles
    s.t = t;
  }
  seq_clip(a, x, s);
  return s;
}
template <class A>
__device__ __forceinline__ TDesc seq_desc(const A& a, const Seq& s) {
  TDesc d;
  d.valid = s.blk < a.nblk;
  d.rel = s.rel0 + 64 * s.t;
  const int l = s.lim0 - 64 * s.t;
  d.lim = l < 0 ? 0 : (l > 64 ? 64 : l);
  return d;
}

// ---- per-wave state ---------------------------------------------------------
template <int D, int NW>
struct WaveState {
  using C = Bf16Cfg<D, NW>;
  bf16x8 qf[C::NC];        // Q fragment (B operand of S^T)
  f32x16 oacc[C::NDT];     // O^T accumulators (unnormalised u)
  float m_ref;             // reference (base 2), -inf before any visible key
  float m_use;             // reference the exponentials subtract (0 while -inf)
  float m_true;            // exact running max (base 2; row-max path only)
  float l_run;             // sum of bf16(2^(s - m_ref)) over the row (both lane halves)
  bf16x8 sel;              // 0/1 selector, A operand of the row sums (see HalfSoftmax)
  unsigned kaddr[C::NC];   // LDS byte address of the K operand reads (buffer 0)
  unsigned vaddr[C::NDT];  // LDS byte address of the V operand reads (buffer 0)
  int voffk[C::DMA];       // copy source offsets (K) within a tile
  int voffv[C::DMA];       // copy source offsets (V) within a tile
};

// Copy the K and V tile under cursor s into LDS at byte offsets kdst and
// vdst of smem; this wave copies C::DMA KiB of each.
template <int D, int NW>
__device__ __forceinline__ void copy_tile(const Seq& s, int HD2, int wave, const int* voffk,
                                          const int* voffv, char* smem, int kdst, int vdst) {
  using C = Bf16Cfg<D, NW>;
  const int kt0 = s.t * C::BC;
  const int rows = min(C::BC, s.len - kt0);
  const int nrec = (rows - 1) * HD2 + D * 2;
  const long long off = (long long)kt0 * HD2;
  __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(s.kp + off), 0, nrec, kRsrcWord3);
  __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(s.vp + off), 0, nrec, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < C::DMA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rk, (lds_void_ptr)(smem + kdst + (wave * C::DMA + i) * 1024), 16, voffk[i], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < C::DMA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (lds_void_ptr)(smem + vdst + (wave * C::DMA + i) * 1024), 16, voffv[i], 0, 0, 0);
}

// Mask of tile (rel, lim) on one score tile s: key j of the tile is masked
// for this lane's query when j >= lim (padding / past the block) or, causal,
// when its position exceeds the query's ([RA] §3.4 diagonal tiles).
__device__ __forceinline__ bool tile_needs_mask(const TDesc& d, bool causal) {
  return d.lim < 64 || (causal && d.rel > -63);
}
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], const TDesc& d, bool causal, int col,
                                          int half) {
  int t = d.lim - 1 - 4 * half;
  if (causal) {
    // query col sees key j when j <= col - rel (rel clamped: only |rel| < 128
    // can cut a tile)
    const int rel = d.rel < -128 ? -128 : (d.rel > 128 ? 128 : d.rel);
    t = min(t, max(-1, col - rel - 4 * half));
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (32 * kt + 8 * (v >> 2) + (v & 3) > t) s[kt][v] = -INFINITY;
}

// Row max of a (masked) score tile in the base-2 domain.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2], float c_scale) {
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
  return pair_max(mx) * c_scale;
}

// Move the reference of the lanes whose max mx exceeds it by more than the
// slack; returns alpha (1 for lanes that keep theirs).  u must be rescaled
// by alpha by the caller, after every product of the old reference.
__device__ __forceinline__ float move_reference(float& m_ref, float& l_run, float mx) {
  const bool need = mx > m_ref + kRescaleSlack;
  const float alpha = need ? fast_exp2(m_ref - mx) : 1.0f;
  l_run *= alpha;
  m_ref = need ? mx : m_ref;
  return alpha;
}

// Softmax of one half (score tile KT: keys 32 KT .. 32 KT + 31) as a
// software pipeline over 8 pairs of scores: time T shifts and scales pair T,
// exponentiates pair T-1, and packs pair T-2 to bf16 (10 time steps).  The
// packed pair is dword pair % 4 of fragment pair / 4 of the half; the two
// fragments are built fresh (not as updates of the previous tile's
// registers, which would keep those alive) and stored to P fragments 2 KT,
// 2 KT + 1 as they complete.
//
// Row sums on the matrix cores.  l adds the bf16-rounded weights that enter
// P V, so that O stays an exact convex combination of V rows.  Each
// completed fragment (16 keys x 32 queries, lane L holding 8 keys of query
// L % 32) is the B operand of one v_mfma_f32_16x16x32_bf16 whose A operand
// is a 0/1 selector: B lane L sits in k-group L / 16 and column L % 16, so
// k-groups of odd index hold queries 16 .. 31 and even ones queries 0 .. 15;
// A row i selects the k-groups of the parity of i / 4.  Output lane L holds
// rows 4 (L / 16) .. + 3 of column L % 16, i.e. the sum over all 16 keys of
// exactly its own query L % 32, in every one of its four registers, already
// combined over the two lane halves.  Two such ops per half replace 32
// vector instructions (unpacking each pair by a mask and a shift, two fp32
// adds); the products by 0 and 1 are exact and the accumulation is fp32.
// A 0 x inf product of an overflowed weight of the partner query gives NaN,
// which the bound checks below treat like an overflow of the lane's own.
struct HalfSoftmax {
  float x[3][2];
  f32x4 ls;  // running sum of the half's completed fragments (16x16x32 output)
  u32x4 g[2];
};
template <int KT, int T>
__device__ __forceinline__ void half_softmax_step(HalfSoftmax& hs, const f32x16& s, float c,
                                                  float nm, const bf16x8& sel, bf16x8 (&pb)[4]) {
  if constexpr (T < 8) {
    hs.x[T % 3][0] = fmaf(s[2 * T], c, nm);
    hs.x[T % 3][1] = fmaf(s[2 * T + 1], c, nm);
  }
  if constexpr (T >= 1 && T - 1 < 8) {
    hs.x[(T - 1) % 3][0] = fast_exp2(hs.x[(T - 1) % 3][0]);
    hs.x[(T - 1) % 3][1] = fast_exp2(hs.x[(T - 1) % 3][1]);
  }
  if constexpr (T >= 2 && T - 2 < 8) {
    constexpr int p = T - 2, g = p / 4, e = 2 * (p % 4);
    const bf16x2 pr = {(__bf16)hs.x[p % 3][0], (__bf16)hs.x[p % 3][1]};
    unsigned d;
    __builtin_memcpy(&d, &pr, 4);
    // pin the pair's work to this slot: without a use here the compiler
    // sinks it out of the matrix phase it fills
    asm volatile("" : "+v"(d));
    hs.g[g][e / 2] = d;
    if constexpr (p % 4 == 3) {
      pb[2 * KT + g] = __builtin_bit_cast(bf16x8, hs.g[g]);
      hs.ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[2 * KT + g],
                                                      g == 0 ? f32x4{} : hs.ls, 0, 0, 0);
    }
  }
}
constexpr int kSoftSteps = 10;

// The half-softmax time steps that go after matrix op i of n.
template <int I, int N>
struct SoftSlot {
  static constexpr int lo = I * kSoftSteps / N, hi = (I + 1) * kSoftSteps / N;
};

template <int KT, int LO, int HI>
__device__ __forceinline__ void half_softmax_range(HalfSoftmax& hs, const f32x16& s, float c,
                                                   float nm, const bf16x8& sel, bf16x8 (&pb)[4]) {
  static_for<LO, HI>([&](auto tc) {
    half_softmax_step<KT, decltype(tc)::value>(hs, s, c, nm, sel, pb);
  });
}

// Both halves of a tile's softmax without matrix work (prologue, the rare
// redo, and phases whose matrix side is idle).
template <int KT>
__device__ __forceinline__ float half_softmax_all(const f32x16& s, float c, float m_use,
                                                  const bf16x8& sel, bf16x8 (&pb)[4]) {
  HalfSoftmax hs;
  half_softmax_range<KT, 0, kSoftSteps>(hs, s, c, -m_use, sel, pb);
  return hs.ls[0];
}

// Front half of a step: S^T(n+1) = K(n+1) Q^T from the K buffer at LDS
// byte offset koff, interleaved with the second half of tile n's softmax.
// Returns that half's contribution to the row sum.  Both run for every
// step: a tile that is dead for the wave (wholly in its future) reaches
// here fully masked, so its weights are exact zeros, and past the end of
// the sequence the products read a stale buffer whose results are unused.
// Keeping the matrix chains free of branches keeps the accumulators in one
// set of registers.
// KOFF >= 0: the K buffer's byte offset as a constant (koff unused).
// after_first: scalar work (the step's tile copies) issued once the first
// two matrix ops are under way, instead of ahead of them.
template <int D, int NW, int KOFF = -1, class Hook>
__device__ __forceinline__ float step_front(WaveState<D, NW>& w, unsigned koff,
                                            const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                            bf16x8 (&pb)[4], float c, const Hook& after_first) {
  using C = Bf16Cfg<D, NW>;
  constexpr int N = C::NQK;
  constexpr int PF = kOperandLead;
  const float nm = -w.m_use;
  HalfSoftmax hs;
  // op i: score tile kt = i % 2, k-step ci = i / 2 (consecutive ops never
  // depend on each other)
  unsigned kbase[C::NC];
  if constexpr (KOFF < 0) {
#pragma unroll
    for (int ci = 0; ci < C::NC; ++ci) kbase[ci] = w.kaddr[ci] + koff;
  }
  bf16x8 kf[PF + 1];
  auto kread = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (KOFF < 0)
      kf[i % (PF + 1)] = lds_read_b128<(i % 2) * 32 * C::ROWB>(kbase[i / 2]);
    else
      kf[i % (PF + 1)] = lds_read_b128<KOFF + (i % 2) * 32 * C::ROWB>(w.kaddr[i / 2]);
  };
  static_for<0, PF>([&](auto ic) { kread(ic); });
  static_for<0, N>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + PF < N) kread(std::integral_constant<int, i + PF>{});
    constexpr int later = (i + PF < N ? i + PF : N - 1) - i;
    claim_lds<later>(kf[i % (PF + 1)]);
    constexpr int kt = i % 2, ci = i / 2;
    s_nxt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (PF + 1)], w.qf[ci],
                                                        ci == 0 ? f32x16{} : s_nxt[kt], 0, 0, 0);
    half_softmax_range<1, SoftSlot<i, N>::lo, SoftSlot<i, N>::hi>(hs, s_cur[1], c, nm, w.sel, pb);
    if constexpr (i == 1) after_first();
    __builtin_amdgcn_sched_barrier(0);
  });
  return hs.ls[0];
}

// Back half of a step: O^T += V(n)^T P(n)^T from the V buffer at LDS byte
// offset vbuf, interleaved with the first half of tile n+1's softmax.
// Returns that half's contribution to the row sum (unconditional, as above).
// VOFF >= 0: the V buffer's byte offset from buffer 0 as a constant (vbuf
// unused).
template <int D, int NW, int VOFF = -1>
__device__ __forceinline__ float step_back(WaveState<D, NW>& w, unsigned vbuf,
                                           const bf16x8 (&pb)[4], const f32x16 (&s_nxt)[2],
                                           bf16x8 (&pb_nxt)[4], float c) {
  using C = Bf16Cfg<D, NW>;
  constexpr int N = C::NPV;
  constexpr int PF = kOperandLead;
  const float nm = -w.m_use;
  HalfSoftmax hs;
  // fragment j = (G = j / NDT, dt = j % NDT): two 64-bit transposed reads
  // (keys 16G .. 16G+7 and 16G+8 .. 16G+15 of d tile dt); consecutive ops
  // accumulate into different d tiles
  unsigned vbase[C::NDT];
  if constexpr (VOFF < 0) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) vbase[dt] = vbuf + w.vaddr[dt];
  } else {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) vbase[dt] = w.vaddr[dt];
  }
  s16x8 vr[PF + 1];
  auto vread = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int off = (VOFF < 0 ? 0 : VOFF) + (j / C::NDT) * 16 * C::ROWB;
    const s16x4 lo = lds_read_tr16<off>(vbase[j % C::NDT]);
    const s16x4 hi = lds_read_tr16<off + 8 * C::ROWB>(vbase[j % C::NDT]);
    vr[j % (PF + 1)] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  static_for<0, PF>([&](auto jc) { vread(jc); });
  static_for<0, N>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j + PF < N) vread(std::integral_constant<int, j + PF>{});
    // reads issued after fragment j's: those of fragments j+1 .. j+PF
    constexpr int later = 2 * ((j + PF < N ? j + PF : N - 1) - j);
    claim_lds<later>(vr[j % (PF + 1)]);
    bf16x8 vf;
    __builtin_memcpy(&vf, &vr[j % (PF + 1)], 16);
    constexpr int G = j / C::NDT, dt = j % C::NDT;
    w.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[G], w.oacc[dt], 0, 0, 0);
    half_softmax_range<0, SoftSlot<j, N>::lo, SoftSlot<j, N>::hi>(hs, s_nxt[0], c, nm, w.sel, pb_nxt);
    __builtin_amdgcn_sched_barrier(0);
  });
  return hs.ls[0];
}

template <int D, int NW>
__device__ __forceinline__ void scale_o(WaveState<D, NW>& w, float alpha) {
#pragma unroll
  for (int i = 0; i < Bf16Cfg<D, NW>::NDT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) w.oacc[i][v] *= alpha;
}

// Row max of one half (score tile s of 16 values per lane) in base 2.
__device__ __forceinline__ float half_max(const f32x16& s, float c_scale) {
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
  return pair_max(mx) * c_scale;
}

// A half whose weights exceed the bound (a score more than ~20 above the
// reference, or an infinite weight): move the reference of the lanes whose
// half max mx lies above it by the whole number of octaves k that brings
// every weight of the half to at most 1, and scale u, l and the other
// weights already formed against the old reference by 2^-k -- exact, as
// scaling by a power of two commutes with rounding.  Returns 2^-k (1 for
// lanes that keep their reference).
__device__ __forceinline__ float move_reference_octaves(float& m_ref, float& l_run, float mx) {
  const bool need = mx > m_ref;
  const float k = need ? ceilf(mx - m_ref) : 0.0f;
  const float f = fast_exp2(-k);
  m_ref += k;
  l_run *= f;
  return f;
}

__device__ __forceinline__ void scale_p(bf16x8& p, float f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = (__bf16)((float)p[e] * f);
}

// S^T of one tile from the K buffer at KOFF, without interleaved work.
template <int D, int NW, int KOFF>
__device__ __forceinline__ void scores_tile(const WaveState<D, NW>& w, f32x16 (&acc)[2]) {
  using C = Bf16Cfg<D, NW>;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) acc[kt] = f32x16{};
  static_for<0, C::NQK>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    bf16x8 kf = lds_read_b128<KOFF + (i % 2) * 32 * C::ROWB>(w.kaddr[i / 2]);
    claim_lds<0>(kf);
    acc[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, w.qf[i / 2], acc[i % 2], 0, 0, 0);
  });
}

// Per-step context that stays fixed over the loop.
template <class A>
struct StepCtx {
  const A* a;
  SeqCtx x;
  int HD2, wave, col, half, wrows;
  bool causal, rowmax;
  float c;
};

// Set up tile n+1 for its softmax (before its first half runs): mask, and,
// on the row-max path or while some row of the wave has no reference yet,
// the row max and a lazy move of the reference.  Returns alpha for the
// deferred rescale of u (1 when nothing moved) and sets `moved`.
template <int D, int NW, bool ML, class A>
__device__ __forceinline__ float tile_setup(const StepCtx<A>& k, WaveState<D, NW>& w, f32x16 (&s)[2],
                                            const TDesc& d, bool& moved) {
  if (tile_needs_mask(d, k.causal)) mask_tile(s, d, k.causal, k.col, k.half);
  float alpha = 1.0f;
  moved = false;
  if (ML || k.rowmax || __builtin_amdgcn_ballot_w64(w.m_ref == -INFINITY)) {
    const float mx = tile_max(s, k.c);
    if (ML) w.m_true = fmaxf(w.m_true, mx);
    if (__builtin_amdgcn_ballot_w64(mx > w.m_ref + kRescaleSlack)) {
      alpha = move_reference(w.m_ref, w.l_run, mx);
      moved = true;
    }
  }
  w.m_use = w.m_ref == -INFINITY ? 0.0f : w.m_ref;
  return alpha;
}

// First half of a tile over the bound: move the reference, scale u and l
// (every product of the old reference has been issued), redo the half.
template <int D, int NW, class A>
__device__ __forceinline__ void first_half_check(const StepCtx<A>& k, WaveState<D, NW>& w,
                                                 const f32x16& s0, bf16x8 (&pb)[4], float& l1) {
  if (__builtin_amdgcn_ballot_w64(!(l1 <= kTileSumLimit))) {
    const float f = move_reference_octaves(w.m_ref, w.l_run, half_max(s0, k.c));
    scale_o<D, NW>(w, f);
    w.m_use = w.m_ref;
    l1 = half_softmax_all<0>(s0, k.c, w.m_use, w.sel, pb);
  }
}

// One pipeline step.  PAR = n & 1 only swaps the roles of the two score
// and P register sets.  K(n) sits in K buffer kb, K(n+1) in the next one,
// V(n) in V buffer vb; the copies of tile n + LEAD go to K buffer
// kb + LEAD and V buffer vb + LEAD (modulo the buffer counts: K(n)'s or
// K(n-1)'s buffer and V(n-1)'s, read in earlier steps).  FS >= 0: the
// step's place in a loop iteration of KBUF = VBUF steps, which makes every
// buffer index a constant (kb and vb are then unused).  d0, d1, d2 describe
// tiles n, n+1, n+2 (d2 only with LEAD = 3) and cur stands at tile n + LEAD.
template <int D, int NW, bool ML, int PAR, int FS = -1, class A>
__device__ __forceinline__ void pipeline_step(const StepCtx<A>& k, char* smem, WaveState<D, NW>& w,
                                              f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                              bf16x8 (&pb_cur)[4], bf16x8 (&pb_nxt)[4],
                                              float& lsum_cur, float& lsum_nxt, Seq& cur,
                                              TDesc& d0, TDesc& d1, TDesc& d2, int& kb, int& vb) {
  using C = Bf16Cfg<D, NW>;
  static_assert(FS < 0 || C::KBUF == C::VBUF, "constant buffers need equal K and V counts");
  const A& a = *k.a;
  const int kb1 = kb + 1 == C::KBUF ? 0 : kb + 1;  // K(n+1)
  const int kcp = kb + C::LEAD >= C::KBUF ? kb + C::LEAD - C::KBUF : kb + C::LEAD;
  const int vcp = vb == 0 ? C::VBUF - 1 : vb - 1;  // V(n-1)'s buffer = vb + LEAD
  // copies of tile n + LEAD: K first, so that waiting for K leaves V in flight;
  // issued from the front phase once its first matrix ops are under way (the
  // buffers they overwrite were released by the barrier that ended step n-1)
  const TDesc dl = seq_desc(a, cur);
  auto copies = [&]() {
    if (dl.valid)
      copy_tile<D, NW>(cur, k.HD2, k.wave, w.voffk, w.voffv, smem,
                       C::KB + (FS >= 0 ? (FS + C::LEAD) % C::KBUF : kcp) * C::TILE,
                       C::VB + (FS >= 0 ? (FS + C::LEAD) % C::VBUF : vcp) * C::TILE);
  };

  // front: S^T(n+1) with the second half of P(n) (tile n is valid here)
  float l2;
  if constexpr (FS >= 0)
    l2 = step_front<D, NW, C::KB + (FS + 1) % C::KBUF * C::TILE>(w, 0u, s_cur, s_nxt, pb_cur,
                                                                   k.c, copies);
  else
    l2 = step_front<D, NW>(w, C::KB + kb1 * C::TILE, s_cur, s_nxt, pb_cur, k.c, copies);
  {
    // second half over the bound: move the reference, scale u, l and the
    // first half's weights, redo the second half
    if (__builtin_amdgcn_ballot_w64(!(l2 <= kTileSumLimit))) {
      const float f = move_reference_octaves(w.m_ref, w.l_run, half_max(s_cur[1], k.c));
      scale_o<D, NW>(w, f);
      scale_p(pb_cur[0], f);
      scale_p(pb_cur[1], f);
      lsum_cur *= f;
      w.m_use = w.m_ref;
      l2 = half_softmax_all<1>(s_cur[1], k.c, w.m_use, w.sel, pb_cur);
    }
    w.l_run += lsum_cur + l2;
  }

  // back: P(n) V(n) with the first half of P(n+1)
  float alpha = 1.0f;
  bool moved = false;
  if (d1.valid) alpha = tile_setup<D, NW, ML>(k, w, s_nxt, d1, moved);
  if constexpr (FS >= 0)
    lsum_nxt = step_back<D, NW, FS % C::VBUF * C::TILE>(w, 0u, pb_cur, s_nxt, pb_nxt, k.c);
  else
    lsum_nxt = step_back<D, NW>(w, vb * C::TILE, pb_cur, s_nxt, pb_nxt, k.c);
  if (moved) scale_o<D, NW>(w, alpha);  // after every product of the old reference
  if (d1.valid) first_half_check<D, NW>(k, w, s_nxt[0], pb_nxt, lsum_nxt);

  // K(n+2) and V(n+1) (and everything older) landed; the later copies may
  // stay in flight
  if constexpr (C::LEAD == 3) {
    if (dl.valid) wait_vmcnt<3 * C::DMA>();
    else if (d2.valid) wait_vmcnt<C::DMA>();
    else wait_vmcnt<0>();
  } else {
    if (dl.valid) wait_vmcnt<C::DMA>();
    else wait_vmcnt<0>();
  }
  pipeline_barrier();  // everyone's copies landed, everyone done reading
  d0 = d1;
  if constexpr (C::LEAD == 3) {
    d1 = d2;
    d2 = dl;
  } else {
    d1 = dl;
  }
  seq_next(a, k.x, cur);
  kb = kb1;
  vb = vb + 1 == C::VBUF ? 0 : vb + 1;
}

// Accumulate mode: fold this launch's partial of output row `so` (the
// normalised values oacc * inv and log-sum-exp lb) into the running partial
// (a.o fp32, a.lse) with the pairwise combine of the merge kernel
// ([SPD] §四):
//   lse' = logaddexp(lse_acc, lb),  o' = o_acc e^(lse_acc - lse') + o e^(lb - lse')
// and write it back, or with a.o_final the combined output there (bf16 when
// FINAL_BF16).  Lane (col, half) holds features 32dt + 8g + 4half .. +3 of
// the row; both halves read lse_acc before half 0 rewrites it (the write
// depends on the value read).
template <int D, bool FINAL_BF16, class A>
__device__ __forceinline__ void fold_row(const A& a, long long so, int half,
                                         const f32x16 (&oacc)[D / 32], float inv, float lb) {
  constexpr int NDT = D / 32;
  float* oa = (float*)a.o + so * D;
  float4 x[NDT][4];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) x[dt][g] = *(const float4*)(oa + 32 * dt + 8 * g + 4 * half);
  const float la = a.lse[so];
  const float mx = fmaxf(la, lb);
  float wa = 0.0f, wb = 0.0f, lse = -INFINITY;
  if (mx != -INFINITY) {
    const float ea = fast_exp2((la - mx) * kLog2eF);
    const float eb = fast_exp2((lb - mx) * kLog2eF);
    const float sum = ea + eb;
    lse = mx + fast_log2(sum) * kLn2;
    const float r = 1.0f / sum;
    wa = ea * r;
    wb = eb * r;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * half;
      const float4 y = float4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                              oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
      const float4 z = float4{fmaf(x[dt][g].x, wa, y.x * wb), fmaf(x[dt][g].y, wa, y.y * wb),
                              fmaf(x[dt][g].z, wa, y.z * wb), fmaf(x[dt][g].w, wa, y.w * wb)};
      if (!a.o_final) {
        *(float4*)(oa + d) = z;
      } else if constexpr (FINAL_BF16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 t;
        t[0] = (__bf16)z.x; t[1] = (__bf16)z.y; t[2] = (__bf16)z.z; t[3] = (__bf16)z.w;
        *(bf16x4*)((__bf16*)a.o_final + so * D + d) = t;
      } else {
        *(float4*)((float*)a.o_final + so * D + d) = z;
      }
    }
  if (half == 0) a.lse[so] = lse;
}

// One (batch, head, query tile) over tiles [lo, hi) of its visited-tile
// sequence.  slot < 0: the output rows of the tile; otherwise the split
// partial slot (see AttnArgs).  ML: also track the exact max for m / l.
template <int D, int NW, bool ML, class A>
__device__ __forceinline__ void attn_bf16_tile(const A& a, char* smem, int b, int h,
                                               int qt, int lo, int hi, long long slot,
                                               int rot = 0) {
  using C = Bf16Cfg<D, NW>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int row0 = qt * C::BR;
  const int rows_here = min(C::BR, a.Sq - row0);
  const int wrow0 = row0 + wave * 32;
  const long long HD = (long long)a.H * D;
  const int hk = h / (a.H / a.Hkv);  // K/V head of this query head

  StepCtx<A> k;
  k.a = &a;
  k.HD2 = a.Hkv * D * 2;  // bytes between consecutive key rows
  k.wave = wave;
  k.col = col;
  k.half = half;
  k.wrows = min(32, a.Sq - wrow0);
  k.causal = a.causal != 0;
  k.rowmax = a.rowmax != 0;
  k.c = a.scale_log2;
  k.x.q_hi = qpos(a, row0 + rows_here - 1);
  k.x.wq_lo = qpos(a, wrow0);
  k.x.boff = ((long long)b * a.kv_rows_b * a.Hkv + hk) * (D * 2);
  k.x.end_blk = a.nblk;
  k.x.end_t = 0;
  k.x.rot = rot;
  if (hi != INT_MAX) seq_locate(a, k.x, hi, k.x.end_blk, k.x.end_t);

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
    w.voffk[i] = r * k.HD2 + swz_k<D>(r, pc) * 16;
    w.voffv[i] = r * k.HD2 + swz_v<D>(r, pc) * 16;
  }
  const unsigned lds0 = (unsigned)(size_t)(lds_void_ptr)smem;
#pragma unroll
  for (int c = 0; c < C::NC; ++c)
    w.kaddr[c] = lds0 + col * C::ROWB + swz_k<D>(col, 2 * c + half) * 16;
  {
    const int j = lane & 15, e = j >> 2, q = j & 3, g = lane >> 4;
    const int kl = 4 * half + e;  // supplier row within a 16-key group
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * q;
      w.vaddr[dt] = lds0 + C::VB + kl * C::ROWB + swz_v<D>(kl, d0 >> 3) * 16 + (d0 & 7) * 2;
    }
  }
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) w.oacc[i] = f32x16{};
  w.m_ref = -INFINITY;
  w.m_use = 0.0f;
  w.m_true = -INFINITY;
  w.l_run = 0.0f;
  {
    // A row lane % 16 in k-group lane / 16: 1 where the parities of the
    // k-group and of row / 4 agree
    const __bf16 one = (((lane >> 4) ^ (lane >> 2)) & 1) ? (__bf16)0.0f : (__bf16)1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) w.sel[e] = one;
  }

  // prologue: tiles 0 .. LEAD-1 into K and V buffers 0 .. LEAD-1; scores of
  // tile 0 and the first half of its softmax
  Seq cur = seq_first(a, k.x, lo);
  TDesc d0 = seq_desc(a, cur), d1{}, d2{};
  static_for<0, C::LEAD>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    const TDesc d = seq_desc(a, cur);
    if (d.valid)
      copy_tile<D, NW>(cur, k.HD2, wave, w.voffk, w.voffv, smem, C::KB + t * C::TILE,
                       C::VB + t * C::TILE);
    if constexpr (t == 1) d1 = d;
    if constexpr (t == 2) d2 = d;
    seq_next(a, k.x, cur);
  });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sA[2], sB[2];
  bf16x8 pA[4], pB[4];
  float lA = 0.0f, lB = 0.0f;
  if (d0.valid) {
    scores_tile<D, NW, C::KB>(w, sA);
    bool moved;
    tile_setup<D, NW, ML>(k, w, sA, d0, moved);
    lA = half_softmax_all<0>(sA[0], k.c, w.m_use, w.sel, pA);
    first_half_check<D, NW>(k, w, sA[0], pA, lA);
  }
  __syncthreads();  // every wave is done with tile 0's K before any new copy

  int kb = 0, vb = 0;  // K and V buffers of tile n
  if constexpr (C::FIXED) {
    static_assert(C::KBUF == 4 && C::VBUF == 4, "four steps per iteration");
    while (d0.valid) {
      pipeline_step<D, NW, ML, 0, 0>(k, smem, w, sA, sB, pA, pB, lA, lB, cur, d0, d1, d2, kb, vb);
      if (!d0.valid) break;
      pipeline_step<D, NW, ML, 1, 1>(k, smem, w, sB, sA, pB, pA, lB, lA, cur, d0, d1, d2, kb, vb);
      if (!d0.valid) break;
      pipeline_step<D, NW, ML, 0, 2>(k, smem, w, sA, sB, pA, pB, lA, lB, cur, d0, d1, d2, kb, vb);
      if (!d0.valid) break;
      pipeline_step<D, NW, ML, 1, 3>(k, smem, w, sB, sA, pB, pA, lB, lA, cur, d0, d1, d2, kb, vb);
    }
  } else {
    while (d0.valid) {
      pipeline_step<D, NW, ML, 0>(k, smem, w, sA, sB, pA, pB, lA, lB, cur, d0, d1, d2, kb, vb);
      if (!d0.valid) break;
      pipeline_step<D, NW, ML, 1>(k, smem, w, sB, sA, pB, pA, lB, lA, cur, d0, d1, d2, kb, vb);
    }
  }

  // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
  const float l_tot = w.l_run;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int r = wrow0 + col;
  if (k.wrows > 0 && r < a.Sq) {
    // output row (b, r, h), or row r - row0 of the split partial slot
    const long long so = slot < 0 ? ((long long)b * a.Sq + r) * a.H + h
                                  : slot * C::BR + (r - row0);
    const long long ro = so * D;
    if (a.acc) {
      const float lb = l_tot > 0.0f ? (w.m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      fold_row<D, true>(a, so, half, w.oacc, inv, lb);
      return;
    }
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
      if (ML) {
        if (a.m_out) a.m_out[so] = seen ? w.m_true * kLn2 : -INFINITY;
        if (a.l_out) a.l_out[so] = seen ? l_tot * fast_exp2(w.m_ref - w.m_true) : 0.0f;
      }
    }
  }
}

// Kernel body: one query tile over its whole visited sequence, or (SPLIT)
// one run of it.
template <int D, int NW, bool ML, bool SPLIT, class A>
__device__ __forceinline__ void attn_bf16_body(const A& a, char* smem) {
  using C = Bf16Cfg<D, NW>;
  if constexpr (SPLIT) {
    const int ns = a.nsplit;
    // XCD-contiguous ranges as in tile_coords: the runs of one head's query
    // tiles stay on one XCD and share its K/V stream in L2
    int id = (int)blockIdx.x;
    if ((gridDim.x & 7) == 0) id = (id & 7) * (int)(gridDim.x >> 3) + (id >> 3);
    const int j = id % ns;
    const int tile = id / ns;  // (b*H + h)*n_qtiles + qt
    const int qt = tile % a.n_qtiles, bh = tile / a.n_qtiles;
    const int row_hi = min((qt + 1) * C::BR, a.Sq) - 1;
    const long long q_hi = qpos(a, row_hi);
    int total = 0;
    for (int bi = 0; bi < a.nblk; ++bi) total += tiles_of<64>(a, bi, q_hi);
    const int lo = (int)((long long)total * j / ns), hi = (int)((long long)total * (j + 1) / ns);
    attn_bf16_tile<D, NW, ML>(a, smem, bh / a.H, bh % a.H, qt, lo, hi, (long long)tile * ns + j);
  } else {
    int b, h, qt, rot = 0;
    if (NW != 8 ||
        !tile_coords_lockstep(a, (int)blockIdx.x, (int)gridDim.x, b, h, qt, rot))
      tile_coords(a, b, h, qt);
    attn_bf16_tile<D, NW, ML>(a, smem, b, h, qt, 0, INT_MAX, -1, rot);
  }
}

template <int D, int NW, bool ML>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, NW>::LDS];
  attn_bf16_body<D, NW, ML, false>(a, smem);
}

// The split ring (AttnArgs.nsplit > 1).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16_split(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, 4>::LDS];
  attn_bf16_body<D, 4, false, true>(a, smem);
}

// Several independent problems in one launch (the packed samples of a
// share): each segment's arguments exactly as its own launch would take
// them (same waves per workgroup; a smaller block table), so that the
// workgroups of all segments fill the chip together instead of each launch
// draining its last, partial round before the next begins.  Workgroups are
// dispatched round-robin over the 8 XCDs: XCD x walks the segments in turn
// and takes the x-th contiguous eighth of each one's tiles (neighbouring
// tiles of the same heads, which share K/V in its L2), so every XCD gets an
// equal share of every segment.  Each segment's workgroup count is padded to
// a multiple of 8; padding workgroups return at once.
constexpr int kMaxSeg = 8, kSegBlk = 8;
using SegProblem = AttnArgsT<kSegBlk>;
struct SegArgs {
  int nseg;
  int c8[kMaxSeg + 1];  // workgroups per XCD before segment s (cumulative)
  SegProblem seg[kMaxSeg];
};
static_assert(sizeof(SegArgs) <= 4096, "kernel arguments of one launch");

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16_seg(const SegArgs sa) {
  __shared__ __attribute__((aligned(1024))) char smem[Bf16Cfg<D, NW>::LDS];
  const int x = (int)blockIdx.x & 7, kx = (int)blockIdx.x >> 3;
  int sg = 0;
  while (sg + 1 < sa.nseg && kx >= sa.c8[sg + 1]) ++sg;
  const SegProblem& a = sa.seg[sg];
  const int per = sa.c8[sg + 1] - sa.c8[sg];  // this segment's workgroups per XCD
  const int j = x * per + (kx - sa.c8[sg]);
  if (j >= a.B * a.H * a.n_qtiles) return;  // padding
  int b, h, qt;
  tile_coords_in(a, j, b, h, qt);
  attn_bf16_tile<D, NW, false>(a, smem, b, h, qt, 0, INT_MAX, -1);
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
    if (a.acc) {
      const float lb = l_tot > 0.0f ? (st.m + fast_log2(l_tot)) * kLn2 : -INFINITY;
      fold_row<D, false>(a, ((long long)b * a.Sq + r) * a.H + h, half, oacc, inv, lb);
      return;
    }
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
// Waves per bf16 workgroup (RA_OPT_ATTN_WAVES): 8 (256 query rows sharing
// one K/V stream, half the copies per FLOP) once that still gives every
// compute unit a workgroup, else 4 (128 rows, two workgroups per compute
// unit).
int bf16_waves(const AttnArgs& a) {
  const int forced = ra::option(RA_OPT_ATTN_WAVES);
  if (forced == 4 || forced == 8) return forced;
  const long long wg8 = (long long)a.B * a.H * ((a.Sq + 255) / 256);
  return wg8 >= 256 ? 8 : 4;
}

template <int D, int NW>
void launch_bf16(const AttnArgs& a, bool ml, dim3 grid, hipStream_t stream) {
  if (ml) hipLaunchKernelGGL((ring_attn_bf16<D, NW, true>), grid, dim3(64 * NW), 0, stream, a);
  else hipLaunchKernelGGL((ring_attn_bf16<D, NW, false>), grid, dim3(64 * NW), 0, stream, a);
}

ra_status launch(AttnArgs& a, int D, ra_dtype dt, hipStream_t stream, const char* name) {
  const bool split = a.nsplit > 1;
  // a split ring keeps 128-row workgroups (its partial slots hold 128 rows)
  const int nw = dt == RA_BF16 && !split ? bf16_waves(a) : 4;
  const int br = 32 * nw;
  a.n_qtiles = (a.Sq + br - 1) / br;
  a.rowmax = ra::option(RA_OPT_ATTN_KERNEL) == RA_KERNEL_ROWMAX;
  const long long n_wg = (long long)a.B * a.H * a.n_qtiles * (split ? a.nsplit : 1);
  if (n_wg == 0) return RA_OK;
  if (n_wg > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: too many query tiles", name);
  for (int i = 0; i < a.nblk; ++i)
    if (a.blk[i].len > (1 << 30))
      return ra::fail(RA_ERR_UNSUPPORTED, "%s: K/V block of %d rows (at most 2^30)", name,
                      a.blk[i].len);
  const dim3 grid((unsigned)n_wg);
  if (split) {
    a.lockstep = 0;
  } else if (a.lockstep == 0) {  // not preset by the caller (the zigzag share)
    a.lockstep = 1;
    for (int i = 1; i < a.nblk; ++i)
      if (a.blk[i].cls != RA_FULL) a.lockstep = 0;
  }
  if (dt == RA_BF16) {
    // m and l are tracked only when asked for
    const bool ml = a.m_out != nullptr || a.l_out != nullptr;
    if (split) {
      if (D == 128) hipLaunchKernelGGL(ring_attn_bf16_split<128>, grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(ring_attn_bf16_split<64>, grid, dim3(256), 0, stream, a);
    } else if (nw == 8) {
      if (D == 128) launch_bf16<128, 8>(a, ml, grid, stream);
      else launch_bf16<64, 8>(a, ml, grid, stream);
    } else {
      if (D == 128) launch_bf16<128, 4>(a, ml, grid, stream);
      else launch_bf16<64, 4>(a, ml, grid, stream);
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

// bf16 problems of one head dimension in as few launches as possible:
// kMaxSeg per launch, in the order given, all with the same waves per
// workgroup (the choice bf16_waves makes for their workgroups together); a
// problem with more than kSegBlk visited blocks takes a launch of its own.
ra_status launch_segments(const AttnArgs* segs, int n, int D, hipStream_t stream,
                          const char* name) {
  long long wg8 = 0;
  for (int i = 0; i < n; ++i) wg8 += (long long)segs[i].B * segs[i].H * ((segs[i].Sq + 255) / 256);
  const int forced = ra::option(RA_OPT_ATTN_WAVES);
  const int nw = forced == 4 || forced == 8 ? forced : wg8 >= 256 ? 8 : 4;
  const int br = 32 * nw;
  const int rowmax = ra::option(RA_OPT_ATTN_KERNEL) == RA_KERNEL_ROWMAX;
  SegArgs sa{};
  long long total = 0;  // workgroups per XCD so far
  auto flush = [&]() -> ra_status {
    if (sa.nseg == 0) return RA_OK;
    sa.c8[sa.nseg] = (int)total;
    if (total > 0) {
      const dim3 grid((unsigned)(8 * total)), blk(64 * nw);
      if (nw == 8) {
        if (D == 128) hipLaunchKernelGGL((ring_attn_bf16_seg<128, 8>), grid, blk, 0, stream, sa);
        else hipLaunchKernelGGL((ring_attn_bf16_seg<64, 8>), grid, blk, 0, stream, sa);
      } else {
        if (D == 128) hipLaunchKernelGGL((ring_attn_bf16_seg<128, 4>), grid, blk, 0, stream, sa);
        else hipLaunchKernelGGL((ring_attn_bf16_seg<64, 4>), grid, blk, 0, stream, sa);
      }
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess)
        return ra::fail(RA_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(err));
    }
    sa = SegArgs{};
    total = 0;
    return RA_OK;
  };
  for (int i = 0; i < n; ++i) {
    const AttnArgs& s = segs[i];
    if (s.nblk > kSegBlk) {  // rare: more visited blocks than a table entry holds
      AttnArgs own = s;
      const ra_status st = launch(own, D, RA_BF16, stream, name);
      if (st != RA_OK) return st;
      continue;
    }
    for (int bi = 0; bi < s.nblk; ++bi)
      if (s.blk[bi].len > (1 << 30))
        return ra::fail(RA_ERR_UNSUPPORTED, "%s: K/V block of %d rows (at most 2^30)", name,
                        s.blk[bi].len);
    const long long wgs = (long long)s.B * s.H * ((s.Sq + br - 1) / br);
    const long long per = (wgs + 7) / 8;
    if (sa.nseg == kMaxSeg || 8 * (total + per) > 0x7fffffffLL) {
      const ra_status st = flush();
      if (st != RA_OK) return st;
    }
    if (8 * per > 0x7fffffffLL) return ra::fail(RA_ERR_UNSUPPORTED, "%s: too many query tiles", name);
    SegProblem& a = sa.seg[sa.nseg];
    static_cast<AttnHead&>(a) = static_cast<const AttnHead&>(s);
    for (int bi = 0; bi < s.nblk; ++bi) a.blk[bi] = s.blk[bi];
    a.n_qtiles = (a.Sq + br - 1) / br;
    a.rowmax = rowmax;
    sa.c8[sa.nseg++] = (int)total;
    total += per;
  }
  return flush();
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

extern "C" ra_status ra_block_attn_fwd_acc(const void* q, const void* k, const void* v,
                                           int B, int Sq, int Sk, int H, int D,
                                           ra_dtype dt, float scale, long long q_pos0,
                                           long long k_pos0, int causal,
                                           long long valid_len, float* o_acc,
                                           float* lse_acc, void* o_final, void* stream) {
  static const char* name = "ra_block_attn_fwd_acc";
  ra::clear_error();
  ra_status st = check_common(name, B, Sq, H, D, dt);
  if (st != RA_OK) return st;
  if (Sk < 0) return ra::fail(RA_ERR_SHAPE, "%s: negative Sk", name);
  const long long n_out = (long long)B * Sq * H;
  if (n_out == 0) return RA_OK;
  if (!q || !o_acc || !lse_acc || (Sk > 0 && (!k || !v)))
    return ra::fail(RA_ERR_NULL, "%s: NULL q/k/v/o_acc/lse_acc", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_acc) ||
      !aligned16(o_final))
    return ra::fail(RA_ERR_SHAPE, "%s: q, k, v, o_acc and o_final must be 16-byte aligned",
                    name);
  if (q_pos0 < 0 || k_pos0 < 0)
    return ra::fail(RA_ERR_RANGE, "%s: negative global position", name);
  if (valid_len < 0) valid_len = INT64_MAX;
  AttnArgs a{};
  a.q = q;
  a.o = o_acc;
  a.lse = lse_acc;
  a.acc = 1;
  a.o_final = o_final;
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
  // a block with no visible pair leaves the partial unchanged: no launch
  // unless the combined output is asked for
  if (a.nblk == 0 && !o_final) return RA_OK;
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
  // every sample that meets the rank's rows is its own problem: its rows of
  // the share against the parts of the visited blocks that lie inside the
  // sample, in ring order (a packed sequence never attends across samples).
  // bf16: the problems go to one launch (kMaxSeg at a time), the ones whose
  // last query tile sees the most keys first; fp32: one launch each.
  std::vector<AttnArgs> segs;
  std::vector<long long> seg_work;
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
    if (dt == RA_BF16) {
      segs.push_back(a);
      seg_work.push_back((causal ? r1 : s1) - s0);
      continue;
    }
    st = launch(a, D, dt, (hipStream_t)stream, name);
    if (st != RA_OK) return st;
  }
  if (segs.empty()) return RA_OK;
  std::vector<int> order(segs.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return seg_work[x] > seg_work[y]; });
  std::vector<AttnArgs> sorted;
  sorted.reserve(segs.size());
  for (int i : order) sorted.push_back(segs[i]);
  return launch_segments(sorted.data(), (int)sorted.size(), D, (hipStream_t)stream, name);
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

extern "C" int ra_lockstep_order(int n, int Q, int BH, int later_rot, int* bh, int* qt,
                                 int* rot) {
  ra::clear_error();
  if (n < 0 || Q <= 0 || BH <= 0 || later_rot < 0 || (long long)Q * BH != n) {
    ra::fail(RA_ERR_SHAPE, "ra_lockstep_order: bad sizes (n=%d, Q=%d, BH=%d, later_rot=%d)", n,
             Q, BH, later_rot);
    return -1;
  }
  if (n > 0 && (!bh || !qt || !rot)) {
    ra::fail(RA_ERR_NULL, "ra_lockstep_order: NULL output");
    return -1;
  }
  for (int id = 0; id < n; ++id)
    if (!ra_order::lockstep_coords(id, n, Q, BH, later_rot, bh[id], qt[id], rot[id])) return 0;
  return 1;
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

// ---------------------------------------------------------------------------
// Split ring without allocation: the workspace is a fixed device array
// ---------------------------------------------------------------------------
namespace {
// Partials of the split ring (o and lse slots, as the caller's workspace
// of ra_ring_attn_fwd_split) for callers that cannot allocate.  Every GPU
// the library runs on holds its own copy until the process ends.
constexpr long long kScratchFloats = 8LL << 20;  // 32 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.  In host code the array's name is only
// a stand-in for the symbol, never an address a kernel may be given.
ra_status scratch_ptr(const char* name, float** out) {
  static std::mutex mu;
  static float* ptr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64)
    return ra::fail(RA_ERR_HIP, "%s: no current device (%s)", name, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return ra::fail(RA_ERR_HIP, "%s: scratch address: %s", name, hipGetErrorString(e));
    ptr[dev] = (float*)p;
  }
  *out = ptr[dev];
  return RA_OK;
}
}  // namespace

extern "C" ra_status ra_ring_attn_fwd_split_noalloc(const void* q_r, const void* const* k_blocks,
                                                    const void* const* v_blocks, int B, int Sb,
                                                    int H, int Hkv, int D, int P, int rank,
                                                    ra_dtype dt, float scale, int causal,
                                                    long long valid_len, int nsplit, void* o,
                                                    float* lse_opt, void* stream) {
  static const char* name = "ra_ring_attn_fwd_split_noalloc";
  ra::clear_error();
  if (nsplit < 0) return ra::fail(RA_ERR_RANGE, "%s: nsplit must be >= 0 (got %d)", name, nsplit);
  long long need = 0;
  int ns = 1;
  if (dt == RA_BF16) {
    ns = ra_ring_split_plan(B, Sb, H, D, P, rank, causal, valid_len, nsplit, &need);
    if (ns < 0) return ra::fail(RA_ERR_SHAPE, "%s: %s", name, ra_last_error());
  }
  if (ns <= 1)  // the single pass needs no workspace
    return ring_fwd(name, q_r, k_blocks, v_blocks, B, Sb, H, Hkv, D, P, rank, dt, scale, causal,
                    valid_len, o, lse_opt, stream);
  if (need > kScratchFloats)
    return ra::fail(RA_ERR_RANGE, "%s: %d runs per query tile need %lld floats of workspace; "
                    "the fixed scratch holds %lld (use ra_ring_attn_fwd_split with a workspace)",
                    name, ns, need, kScratchFloats);
  float* ws = nullptr;
  ra_status st = scratch_ptr(name, &ws);
  if (st != RA_OK) return st;
  return ring_fwd(name, q_r, k_blocks, v_blocks, B, Sb, H, Hkv, D, P, rank, dt, scale, causal,
                  valid_len, o, lse_opt, stream, ns, ws, kScratchFloats);
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
  // causal: the table starts with the share's own two chunks (each diagonal
  // for one half of the rows; the test leaves out a chunk that is all
  // padding), so the later query tiles of the lockstep order start from the
  // third entry
  if (causal && a.nblk >= 2 && cls[0] != RA_SKIP && cls[1] != RA_SKIP) a.lockstep = 2;
  return launch(a, D, dt, (hipStream_t)stream, name);
}
