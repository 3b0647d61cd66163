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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
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

// Position in the visited-tile sequence: tile t (of n) of visited block blk.
struct Cursor {
  int blk, t, n;
};

__device__ __forceinline__ Cursor cursor_first(const AttnArgs& a, long long q_hi) {
  Cursor c{0, 0, 0};
  while (c.blk < a.nblk && (c.n = tiles_of<64>(a, c.blk, q_hi)) == 0) ++c.blk;
  return c;
}
__device__ __forceinline__ Cursor cursor_next(const AttnArgs& a, long long q_hi, Cursor c) {
  if (c.blk >= a.nblk) return c;
  if (++c.t < c.n) return c;
  c.t = 0;
  ++c.blk;
  while (c.blk < a.nblk && (c.n = tiles_of<64>(a, c.blk, q_hi)) == 0) ++c.blk;
  return c;
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
// visited block of `len` rows) into LDS at `dst`; each wave copies C::DMA KiB.
template <int D, int NW>
__device__ __forceinline__ void copy_tile(const void* src, int len, int ti, int b, int h,
                                          int H, int HD2, int wave, const int* voff,
                                          char* dst) {
  using C = Bf16Cfg<D, NW>;
  const int kt0 = ti * C::BC;
  const int rows = min(C::BC, len - kt0);
  const long long off = (((long long)b * len + kt0) * H + h) * (D * 2);
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

// One pipeline step.  PAR = n & 1: K(n+1) sits in K buffer PAR^1, V(n) in
// V buffer PAR; the copies go to K buffer PAR and V buffer PAR^1.
template <int D, int NW, int PAR>
__device__ __forceinline__ void pipeline_step(
    const AttnArgs& a, char* smem, WaveState<D, NW>& w, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
    Cursor& t0, Cursor& t1, Cursor& t2, int& vb,
    long long q_hi, long long wq_lo, long long wq_hi, int wrows, int col, int half, int b,
    int h, int HD2, int wave) {
  using C = Bf16Cfg<D, NW>;
  constexpr int BC = C::BC;
  const float c_scale = a.scale_log2;
  // copies of tile n+2: K first, so that waiting for it leaves V in flight
  const int vb2 = vb == 0 ? 2 : vb - 1;  // (vb + 2) % 3
  const bool copy2 = t2.blk < a.nblk;
  if (copy2) {
    const KVBlock& kb2 = a.blk[t2.blk];
    copy_tile<D, NW>(kb2.k, kb2.len, t2.t, b, h, a.H, HD2, wave, w.voffk,
                 smem + C::KB + PAR * C::TILE);
    copy_tile<D, NW>(kb2.v, kb2.len, t2.t, b, h, a.H, HD2, wave, w.voffv,
                 smem + C::VB + vb2 * C::TILE);
  }
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
  bf16x8 pb[C::NS / 8];
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
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + PF < NSTEP) kf[(i + PF) % (PF + 1)] = kread(i + PF);
      const int kt = i % 2, c = i / 2;
      s_nxt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (PF + 1)], w.qf[c],
                                                          c == 0 ? f32x16{} : s_nxt[kt], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < PER; j += 2) {
        const int v = i * PER + j;  // score index, even
        const float e0 = fast_exp2(fmaf(s_cur[v >> 4][v & 15], c_scale, -m_use));
        const float e1 = fast_exp2(fmaf(s_cur[v >> 4][(v & 15) + 1], c_scale, -m_use));
        const int G = 2 * (v >> 4) + ((v & 15) >> 3), e = v & 7;
        pb[G][e] = (__bf16)e0;
        pb[G][e + 1] = (__bf16)e1;
        const bf16x2 pr = {pb[G][e], pb[G][e + 1]};
        lp[(v >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, lp[(v >> 1) & 1], false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    w.l_run += lp[0] + lp[1];
  } else {
    if (live1) scores_tile<D, NW>(smem, kbuf_next, w, s_nxt);
    if (live0) exp_tile(s_cur, m_use, c_scale, pb, w.l_run);
  }
  // O^T += V(n)^T P(n)^T: fragment j = (G = j / NDT, dt = j % NDT) is read
  // two ops ahead, and consecutive ops accumulate into different d tiles
  if (live0) {
    char* vl = smem + C::VB + vb * C::TILE;
    constexpr int NJ = (BC / 16) * C::NDT;
    constexpr int PF = NJ >= 8 ? 4 : 2;
    auto vread = [&](int j) -> bf16x8 {
      char* p0 = vl + (j / C::NDT) * 16 * C::ROWB + w.vaddr[j % C::NDT];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p0 + 8 * C::ROWB));
      bf16x8 vf;
      __builtin_memcpy(&vf, &lo, 8);
      __builtin_memcpy((char*)&vf + 8, &hi, 8);
      return vf;
    };
    bf16x8 vf[PF + 1];
#pragma unroll
    for (int j = 0; j < PF; ++j) vf[j] = vread(j);
    // this phase is matrix-core bound: give it issue priority over the
    // other wave on the SIMD, whose exponentials fill the gaps
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + PF < NJ) vf[(j + PF) % (PF + 1)] = vread(j + PF);
      const int G = j / C::NDT, dt = j % C::NDT;
      w.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j % (PF + 1)], pb[G], w.oacc[dt],
                                                           0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  // this wave's K(n+2) copy (and everything older) landed; V(n+2) may fly
  if (copy2) wait_vmcnt<C::DMA>();
  else wait_vmcnt<0>();
  __syncthreads();  // everyone's copies landed, everyone done reading
  t0 = t1;
  t1 = t2;
  t2 = cursor_next(a, q_hi, t2);
  vb = vb == 2 ? 0 : vb + 1;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ring_attn_bf16(const AttnArgs a) {
  using C = Bf16Cfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  int b, h, qt;
  tile_coords(a, b, h, qt);
  const int row0 = qt * C::BR;
  const int rows_here = min(C::BR, a.Sq - row0);
  const long long q_lo = a.q_pos0 + row0;
  const long long q_hi = q_lo + rows_here - 1;
  const int wrow0 = row0 + wave * 32;
  const int wrows = min(32, a.Sq - wrow0);
  const long long wq_lo = a.q_pos0 + wrow0;
  const long long wq_hi = wq_lo + wrows - 1;
  const long long HD = (long long)a.H * D;
  const int HD2 = a.H * D * 2;  // bytes between consecutive key rows

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

  // prologue: K(0), V(0), K(1) into K0, V0, K1; scores of tile 0
  Cursor t0 = cursor_first(a, q_hi);
  Cursor t1 = cursor_next(a, q_hi, t0);
  Cursor t2 = cursor_next(a, q_hi, t1);
  f32x16 sA[2], sB[2];
  if (t0.blk < a.nblk) {
    const KVBlock& kb = a.blk[t0.blk];
    copy_tile<D, NW>(kb.k, kb.len, t0.t, b, h, a.H, HD2, wave, w.voffk, smem + C::KB);
    copy_tile<D, NW>(kb.v, kb.len, t0.t, b, h, a.H, HD2, wave, w.voffv, smem + C::VB);
  }
  if (t1.blk < a.nblk) {
    const KVBlock& kb = a.blk[t1.blk];
    copy_tile<D, NW>(kb.k, kb.len, t1.t, b, h, a.H, HD2, wave, w.voffk, smem + C::KB + C::TILE);
    copy_tile<D, NW>(kb.v, kb.len, t1.t, b, h, a.H, HD2, wave, w.voffv, smem + C::VB + C::TILE);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t0.blk < a.nblk) {
    const long long kp0 = a.blk[t0.blk].k_pos0 + (long long)t0.t * C::BC;
    if (wrows > 0 && !(a.causal && kp0 > wq_hi)) scores_tile<D, NW>(smem, C::KB, w, sA);
  }
  __syncthreads();  // K buffer 0 is free for K(2)

  int vb = 0;  // V buffer of tile n
  while (t0.blk < a.nblk) {
    pipeline_step<D, NW, 0>(a, smem, w, sA, sB, t0, t1, t2, vb, q_hi, wq_lo, wq_hi, wrows, col,
                        half, b, h, HD2, wave);
    if (t0.blk >= a.nblk) break;
    pipeline_step<D, NW, 1>(a, smem, w, sB, sA, t0, t1, t2, vb, q_hi, wq_lo, wq_hi, wrows, col,
                        half, b, h, HD2, wave);
  }

  // ---- epilogue: o = u / l, lse = m + ln l ([RA] §3.2; [SPD] §四) ----
  const float l_tot = pair_sum(w.l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int r = wrow0 + col;
  if (wrows > 0 && r < a.Sq) {
    const long long ro = ((long long)b * a.Sq + r) * HD + (long long)h * D;
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
      const long long so = ((long long)b * a.Sq + r) * a.H + h;
      const bool seen = l_tot > 0.0f;
      if (a.lse) a.lse[so] = seen ? (w.m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (a.m_out) a.m_out[so] = seen ? w.m_true * kLn2 : -INFINITY;
      if (a.l_out) a.l_out[so] = seen ? l_tot * fast_exp2(w.m_ref - w.m_true) : 0.0f;
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
// Kernel choice for bf16: the 256-row ping-pong kernel halves K/V traffic
// per FLOP; the 128-row kernel runs two workgroups per CU.

int bf16_waves(const AttnArgs& a) {
  const int mode = ra::option(RA_OPT_ATTN_KERNEL);
  if (mode == RA_KERNEL_BR128) return 4;
  if (mode == RA_KERNEL_BR256) return 8;
  // AUTO: the 128-row kernel measured faster on every shape tried (the
  // 256-row one halves the K/V re-reads but keeps its eight waves in step)
  return 4;
}

template <int NW>
void launch_bf16(const AttnArgs& a, int D, dim3 grid, hipStream_t stream) {
  if (D == 128) hipLaunchKernelGGL((ring_attn_bf16<128, NW>), grid, dim3(64 * NW), 0, stream, a);
  else hipLaunchKernelGGL((ring_attn_bf16<64, NW>), grid, dim3(64 * NW), 0, stream, a);
}

ra_status launch(AttnArgs& a, int D, ra_dtype dt, hipStream_t stream, const char* name) {
  const int nw = dt == RA_BF16 ? bf16_waves(a) : kWaves;
  const int br = 32 * nw;
  a.n_qtiles = (a.Sq + br - 1) / br;
  const long long n_wg = (long long)a.B * a.H * a.n_qtiles;
  if (n_wg == 0) return RA_OK;
  if (n_wg > 0x7fffffffLL)
    return ra::fail(RA_ERR_UNSUPPORTED, "%s: too many query tiles", name);
  const dim3 grid((unsigned)n_wg);
  if (dt == RA_BF16) {
    if (nw == 8) launch_bf16<8>(a, D, grid, stream);
    else launch_bf16<4>(a, D, grid, stream);
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
