/*
 * ringattn.h -- C ABI of the MI355X (gfx950) ring-order block attention and
 * Ulysses layout library (libringattn.so).
 *
 * What it computes: exact scaled dot-product attention O = softmax(Q K^T *
 * scale) V (scale = 1/sqrt(D) by default, D the head dimension) for ONE
 * rank's share of a sequence-parallel job, evaluated the Ring-Attention way:
 * the rank's query shard stays put while the P key/value blocks are visited
 * in ring order and merged by the online-softmax recurrence, plus the Ulysses
 * sequence-shard <-> head-shard transposes as local permutations.
 *
 * Pages cited (by title and section):
 *   [RA]  "序列并行与 Ring Attention" (Sequence Parallelism and Ring Attention
 *         tutorial, jefxiong.cn): §3.1 attention and the rank-local output,
 *         §3.2 online softmax (m, l, u, alpha), §3.3 ring order, §3.4 causal
 *         block classes on global positions, §3.5 Ulysses transpose.
 *   [SPD] juejin post 7702110021828427786 (a sequence-parallel attention
 *         library that never communicated): §三 the (B, S_local, H, D) call
 *         shape, §四 the log-sum-exp combine and the is_causal precondition.
 *   [UG]  "Finalize guidelines for Ulysses-based context-parallel attention"
 *         (aitangshan.cn): §三-§七 divisibility and padding.
 *
 * Conventions for every entry point:
 *   - Activations are [B, S, H, D] row-major, D innermost, contiguous
 *     (the shards are made contiguous before the call, [SPD] §三).
 *   - Device pointers are plain HIP device addresses owned by the caller;
 *     the library never allocates, frees or keeps them.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream); work is enqueued
 *     there and is asynchronous to the host.
 *   - Validation happens on the host before anything is launched; on error
 *     nothing is enqueued, a status != RA_OK is returned and
 *     ra_last_error() (thread-local) describes it.  A launch failure returns
 *     RA_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation.  Nothing aborts or throws across the ABI.
 *   - Global positions: query row i of a call sits at q_pos0 + i, key row j
 *     at k_pos0 + j.  Keys at positions >= valid_len are padding and masked
 *     (valid_len < 0 means "no padding").  Causal attention lets query i see
 *     key j only when pos(j) <= pos(i) ([RA] §3.4, §09: global, not local,
 *     indices).  A query that sees no key gets O = 0, lse = -inf.
 *   - Supported: D in {64, 128}; dtype bf16 (fp32 accumulation) or fp32.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL */
  RA_ERR_SHAPE = 2,       /* sizes inconsistent (e.g. S not divisible by P) */
  RA_ERR_DTYPE = 3,       /* unknown dtype / element size */
  RA_ERR_RANGE = 4,       /* an index out of range (rank >= P, P > RA_MAX_P) */
  RA_ERR_UNSUPPORTED = 5, /* valid but not implemented (e.g. D = 96) */
  RA_ERR_HIP = 6          /* the HIP runtime refused a launch */
} ra_status;

typedef enum { RA_BF16 = 0, RA_FP32 = 1 } ra_dtype;

/* Block classes of [RA] §3.4: a K/V block wholly in the future of the query
 * block is skipped, one wholly in the past needs no mask, the overlapping
 * (diagonal) one gets the element mask. */
typedef enum { RA_SKIP = 0, RA_FULL = 1, RA_DIAG = 2 } ra_block_class;

#define RA_MAX_P 64          /* largest ring degree one call accepts */
#define RA_PAD_MULTIPLE 16   /* default per-rank padding granularity */

/* Process-wide options (ra_set_option). */
typedef enum { RA_OPT_ATTN_KERNEL = 0, RA_OPT_ATTN_WAVES = 1, RA_OPT_COUNT = 2 } ra_option;
/* Values of RA_OPT_ATTN_KERNEL: how the bf16 attention kernels keep the
 * per-row reference max of the online softmax ([RA] §3.2).  Both compute
 * the same function to the same tolerance (u and l always share the
 * reference, so u / l does not depend on it).
 *   RA_KERNEL_AUTO (default): a row's reference is its exact max on its
 *     first tile with a visible key; later tiles skip the row max, and a
 *     tile whose weights exceed 2^20 is redone against its own max.
 *   RA_KERNEL_ROWMAX: the row max of every tile is taken and the reference
 *     moved when the max exceeds it by more than 8 (base-2 units).
 * The ROWMAX path also runs whenever m and l are requested.  Any other
 * value is rejected by ra_set_option. */
#define RA_KERNEL_AUTO 0
#define RA_KERNEL_ROWMAX 1
/* Values of RA_OPT_ATTN_WAVES: waves (of 32 query rows) per workgroup of
 * the bf16 attention kernels.  0 (default) picks 8 -- 256 query rows that
 * share one K/V stream, one workgroup per compute unit -- when the share
 * still gives every compute unit a workgroup, else 4 (128 rows, two
 * workgroups per compute unit).  4 or 8 force that count; the split ring
 * always uses 4.  Results are the same to the stated tolerance.  The
 * backward's dQ kernel follows the same rule and setting (its result does
 * not depend on it, bit for bit).  Any other value is rejected by
 * ra_set_option. */

/* ---------------------------------------------------------------------
 * Host-only helpers (no GPU needed; exported for tests and schedule dumps)
 * ------------------------------------------------------------------- */

/* ABI version of this header (bumped on any signature change). */
int ra_abi_version(void);

/* Set a process-wide option (ra_option) to `value`; takes effect for
 * launches made after the call (all threads).  RA_ERR_RANGE for an unknown
 * option or value.  ra_get_option returns the current value. */
ra_status ra_set_option(int option, int value);
int ra_get_option(int option);

/* Message of the last error on the calling thread ("" if none).  The
 * pointer stays valid until the next ra_* call on this thread. */
const char* ra_last_error(void);

/* Padded global length: the smallest multiple of P * pad_multiple that is
 * >= S ([UG] §六 padded_seq_len; its §七 test pads 3000 to 3008 for four
 * ranks, which holds with pad_multiple = RA_PAD_MULTIPLE).  Returns -1 (and
 * sets the error) if S < 0, P <= 0 or pad_multiple <= 0. */
long long ra_padded_len(long long S, int P, int pad_multiple);

/* Rank `rank`'s contiguous shard [*begin, *end) = [rank*S/P, (rank+1)*S/P)
 * of a length-S sequence ([SPD] §三 shard-cover check).  RA_ERR_SHAPE if
 * S % P != 0 (the message names the padded length), RA_ERR_RANGE if rank is
 * outside [0, P). */
ra_status ra_shard_range(long long S, int P, int rank, long long* begin,
                         long long* end);

/* Class of query positions [q0, q1) against key positions [k0, k1)
 * ([RA] §3.4), written to *cls as an ra_block_class.  Non-causal blocks are
 * FULL unless padding keys (>= valid_len) are involved. */
ra_status ra_classify_block(long long q0, long long q1, long long k0,
                            long long k1, int causal, long long valid_len,
                            int* cls);

/* The ring of rank `rank` among P ranks with blocks of block_len rows:
 * src_out[t] = (rank - t) mod P for t = 0..P-1 ([RA] §3.3) and
 * class_out[t] = the class of that block against the rank's query shard.
 * Both arrays are caller-owned host arrays of P ints. */
ra_status ra_ring_schedule(int P, int rank, long long block_len, int causal,
                           long long valid_len, int* src_out, int* class_out);

/* Zigzag (load-balanced causal) sharding ([RA] §3.4: with contiguous shards
 * a causal ring gives rank r about r+1/2 blocks of work; holding an early
 * and a late part of the sequence on every rank balances it).  Reading
 * adopted: the padded sequence is cut into 2P chunks of chunk_len rows and
 * rank r holds chunk r followed by chunk 2P-1-r.  Every rank then has
 * chunk_len * (2P * chunk_len + 1) visible (query, key) pairs per head when
 * causal.
 *
 * ra_zigzag_padded_len: the smallest multiple of 2P * 64 that is >= S (the
 * kernels need chunks of a multiple of 64 rows); -1 and the error set if
 * S < 0 or P <= 0.
 *
 * ra_zigzag_schedule: src_out[t] = (rank - t) mod P for t = 0..P-1 (the ring
 * order of [RA] §3.3 over the ranks' shares) and class_out[2t + h] = the
 * class of chunk (h == 0 ? src : 2P-1-src) against the positions from the
 * rank's first to its last query (SKIP: after every query; FULL: before
 * every query and all real).  src_out holds P ints, class_out 2P ints,
 * both caller-owned host arrays.  Errors: RA_ERR_NULL, RA_ERR_SHAPE,
 * RA_ERR_RANGE (rank outside [0, P)). */
long long ra_zigzag_padded_len(long long S, int P);
ra_status ra_zigzag_schedule(int P, int rank, long long chunk_len, int causal,
                             long long valid_len, int* src_out, int* class_out);

/* ---------------------------------------------------------------------
 * Device entry points
 * ------------------------------------------------------------------- */

/* One round of the ring: attention of the query shard q [B,Sq,H,D] over ONE
 * key/value block k, v [B,Sk,H,D] (both in dtype dt), at global positions
 * q_pos0 / k_pos0 ([SPD] §四 local_attn_with_lse; [RA] §3.2 block step).
 * Outputs (device, fp32, caller-owned):
 *   o   [B,Sq,H,D]  this block's normalised partial output;
 *   lse [B,Sq,H]    natural log-sum-exp of the visible scaled scores;
 *   m_opt [B,Sq,H]  max of the visible scaled scores (may be NULL);
 *   l_opt [B,Sq,H]  sum of exp(score - m) (may be NULL).
 * scale <= 0 selects 1/sqrt(D).  Rows with no visible key: o = 0,
 * lse = m = -inf, l = 0.  Errors: RA_ERR_NULL, RA_ERR_SHAPE (negative
 * sizes), RA_ERR_UNSUPPORTED (D not 64/128), RA_ERR_DTYPE, RA_ERR_HIP. */
ra_status ra_block_attn_fwd(const void* q, const void* k, const void* v,
                            int B, int Sq, int Sk, int H, int D, ra_dtype dt,
                            float scale, long long q_pos0, long long k_pos0,
                            int causal, long long valid_len, float* o,
                            float* lse, float* m_opt, float* l_opt,
                            void* stream);

/* One ring round folded into the running result in the same launch ([RA]
 * §3.2 block step followed by the [SPD] §四 combine of ra_ring_merge): the
 * attention of q over the block k, v exactly as ra_block_attn_fwd computes
 * it, then, per row, with lse_b its log-sum-exp and o_b its normalised
 * output,
 *   lse' = logaddexp(lse_acc, lse_b)
 *   o'   = o_acc * exp(lse_acc - lse') + o_b * exp(lse_b - lse')
 * o_acc [B,Sq,H,D] and lse_acc [B,Sq,H] (device, fp32, caller-owned) must
 * hold a valid partial: the output of ra_block_attn_fwd or of an earlier
 * call, or o = 0 / lse = -inf rows for an empty start.  With o_final NULL
 * the combined partial is written back to o_acc and lse_acc.  Otherwise the
 * combined output goes to o_final [B,Sq,H,D] in dt (the ring's last round:
 * no fp32 copy), lse_acc receives the final log-sum-exp and o_acc is not
 * written.  A block with no visible pair ([RA] §3.4 SKIP) leaves the
 * partial as it is (no launch unless o_final is given).  Positions, causal,
 * valid_len and scale as ra_block_attn_fwd.  Errors: those of
 * ra_block_attn_fwd (o_acc, lse_acc in place of o, lse; o_final must be
 * 16-byte aligned). */
ra_status ra_block_attn_fwd_acc(const void* q, const void* k, const void* v,
                                int B, int Sq, int Sk, int H, int D, ra_dtype dt,
                                float scale, long long q_pos0, long long k_pos0,
                                int causal, long long valid_len, float* o_acc,
                                float* lse_acc, void* o_final, void* stream);

/* Fold one round's partial into the running result ([SPD] §四 combine):
 *   lse' = logaddexp(lse_acc, lse_blk)
 *   o'   = o_acc * exp(lse_acc - lse') + o_blk * exp(lse_blk - lse')
 * in place in o_acc [B,Sq,H,D] / lse_acc [B,Sq,H] (fp32).  Two empty
 * partials (lse = -inf) merge to (0, -inf), never NaN.  If o_final_opt is
 * not NULL, o' is also written there in final_dt ([B,Sq,H,D], bf16 by
 * round-to-nearest-even, or fp32).  Errors: RA_ERR_NULL, RA_ERR_SHAPE,
 * RA_ERR_DTYPE, RA_ERR_HIP. */
ra_status ra_ring_merge(float* o_acc, float* lse_acc, const float* o_blk,
                        const float* lse_blk, int B, int Sq, int H, int D,
                        void* o_final_opt, ra_dtype final_dt, void* stream);

/* The whole ring of rank `rank` in one launch ([RA] §3.2-§3.4): the query
 * shard q_r [B,Sb,H,D] (global rows rank*Sb ..) against the P blocks
 * k_blocks[j], v_blocks[j] (each [B,Sb,H,D], global rows j*Sb ..), visited
 * in the order (rank - t) mod P, future blocks (causal) never read, the
 * running (m, l, u) kept on chip across rounds.  k_blocks / v_blocks are
 * HOST arrays of P device pointers.  Output o [B,Sb,H,D] in dt (bf16 by
 * round-to-nearest-even), lse_opt [B,Sb,H] fp32 natural log-sum-exp (may
 * be NULL).  valid_len: real global length (keys at or beyond it are padding;
 * < 0 means P*Sb).  Errors: RA_ERR_NULL, RA_ERR_SHAPE, RA_ERR_RANGE
 * (rank >= P, P > RA_MAX_P), RA_ERR_UNSUPPORTED, RA_ERR_DTYPE, RA_ERR_HIP. */
ra_status ra_ring_attn_fwd(const void* q_r, const void* const* k_blocks,
                           const void* const* v_blocks, int B, int Sb, int H,
                           int D, int P, int rank, ra_dtype dt, float scale,
                           int causal, long long valid_len, void* o,
                           float* lse_opt, void* stream);

/* Grouped-query form of ra_ring_attn_fwd ([RA] §3.5 and §6 name GQA, where
 * fewer K/V heads than query heads serve groups of query heads): q_r is
 * [B,Sb,H,D], every k_blocks[j] / v_blocks[j] is [B,Sb,H_kv,D], and query
 * head h attends with K/V head h / (H / H_kv).  H_kv = H is the plain ring,
 * H_kv = 1 multi-query attention.  RA_ERR_SHAPE unless H_kv > 0 divides H;
 * everything else as ra_ring_attn_fwd. */
ra_status ra_ring_attn_fwd_gqa(const void* q_r, const void* const* k_blocks,
                               const void* const* v_blocks, int B, int Sb, int H,
                               int H_kv, int D, int P, int rank, ra_dtype dt,
                               float scale, int causal, long long valid_len,
                               void* o, float* lse_opt, void* stream);

/* Split form of ra_ring_attn_fwd / _gqa, for shares too small to fill the
 * chip (B*H*ceil(Sb/128) workgroups of 128 query rows against the device's
 * slots).  The visited-tile sequence of every 128-row query tile (the
 * 64-key tiles of the visited blocks in ring order, [RA] §3.3, up to the
 * last one with a key the tile can see) is cut into nsplit near-equal runs
 * computed by separate workgroups of ONE launch, each leaving a normalised
 * fp32 partial (o, lse) -- the per-round results of [RA] §3.3 grouped --
 * which a second launch merges per row with the log-sum-exp combine of
 * [SPD] §四 (n-way).  Same result as the single pass up to the bf16 rounding
 * of the weights (each run rounds against its own reference max).
 * nsplit >= 1 (RA_ERR_RANGE otherwise); 1, and fp32 inputs, run the single
 * pass with the workspace untouched.  Workspace: caller-owned device fp32
 * of at least ws_floats = B*H*ceil(Sb/128)*nsplit*128*(D+1) floats (what
 * ra_ring_split_plan reports), 16-byte aligned, overwritten (RA_ERR_NULL /
 * RA_ERR_SHAPE otherwise).  H_kv as in ra_ring_attn_fwd_gqa (H_kv = H for
 * the plain ring).  Two launches on `stream`.  Other errors as
 * ra_ring_attn_fwd_gqa. */
ra_status ra_ring_attn_fwd_split(const void* q_r, const void* const* k_blocks,
                                 const void* const* v_blocks, int B, int Sb, int H,
                                 int H_kv, int D, int P, int rank, ra_dtype dt,
                                 float scale, int causal, long long valid_len,
                                 int nsplit, float* ws, long long ws_floats,
                                 void* o, float* lse_opt, void* stream);

/* ra_ring_attn_fwd_split for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result, with the partials in a fixed
 * device array of the library (32 MiB = 8 Mi floats per GPU, held until
 * the process ends) instead of a caller workspace.  nsplit = 0 takes
 * ra_ring_split_plan's choice, nsplit >= 1 that run count (RA_ERR_RANGE for
 * nsplit < 0).  A plan of one run, and fp32 inputs, run the single pass.
 * RA_ERR_RANGE, before any launch, when the plan needs more than 8 Mi
 * floats (ra_ring_split_plan's ws_floats).  Calls no allocating routine.
 * The array is shared by every call on a GPU and keeps the last call's
 * contents; calls that overlap on one GPU (several streams or threads)
 * race and must be serialised by the caller.  Other arguments and errors
 * as ra_ring_attn_fwd_split. */
ra_status ra_ring_attn_fwd_split_noalloc(const void* q_r, const void* const* k_blocks,
                                         const void* const* v_blocks, int B, int Sb, int H,
                                         int H_kv, int D, int P, int rank, ra_dtype dt,
                                         float scale, int causal, long long valid_len,
                                         int nsplit, void* o, float* lse_opt, void* stream);

/* Host-only: the lockstep workgroup order that the 8-wave forward and dQ
 * kernels take for a launch of n = Q * BH workgroups (Q query tiles of 256
 * rows per (batch, head), BH of them), for callers that inspect a schedule
 * and for tests; not needed to call any kernel.  Workgroups are dispatched
 * round-robin over the 8 XCDs (32 CUs each); dispatch index id lands on XCD
 * id % 8.  Each XCD takes whole (batch, head) problems in turn and a head's
 * query tiles in pairs of 32-tile chunks from the top: the later chunk with
 * block-table rotation later_rot (its blocks seen whole first, the diagonal
 * block last), the earlier chunk in decreasing tile order with rotation 0,
 * so that the 32 workgroups of an XCD read each K/V tile at the same step
 * ([RA] §3.3 ring order with §3.4's causal classes; the order of the blocks
 * inside one launch changes only the rounding).  Fills bh[id], qt[id] and
 * rot[id] (HOST arrays of n) and returns 1 when the order applies (n and BH
 * multiples of 8, Q a multiple of 64); returns 0 (arrays partly written) when
 * the kernels keep their plain order for this shape; -1 with RA_ERR_SHAPE
 * when n != Q * BH or a size is not positive, RA_ERR_NULL for a NULL array
 * (message in ra_last_error). */
int ra_lockstep_order(int n, int Q, int BH, int later_rot, int* bh, int* qt, int* rot);

/* Host-only plan of the split ring for this share.  nsplit = 0 chooses:
 * as many runs per query tile as keep the B*H*ceil(Sb/128)*nsplit
 * workgroups within the device's 512 workgroup slots (two 128-row
 * workgroups per compute unit on 256 compute units), each at least 8 tiles
 * of the longest sequence, and 1 (no split) once the single pass fills the
 * slots; nsplit >= 1 plans that count.  Returns the run count (1: the
 * single pass; -1 on bad sizes or rank, message in ra_last_error) and, in
 * *ws_floats (may be NULL), the workspace ra_ring_attn_fwd_split needs for
 * it (0 for the single pass). */
int ra_ring_split_plan(int B, int Sb, int H, int D, int P, int rank, int causal,
                       long long valid_len, int nsplit, long long* ws_floats);

/* Packed variable-length form of ra_ring_attn_fwd ([RA] §6: a packed
 * sequence carries its sample boundaries and a sample never attends to
 * another).  B = 1; the P*Sb global positions hold n_seqs samples, sample i
 * at [cu_seqlens[i], cu_seqlens[i+1]) (a HOST array of n_seqs + 1
 * increasing int64 values from 0; positions past cu_seqlens[n_seqs] are
 * padding).  Query at position p attends to the keys of its own sample
 * (causal: at or before p).  q_r [1,Sb,H,D], blocks [1,Sb,H,D] as in
 * ra_ring_attn_fwd; rows of the share outside every sample are left
 * untouched in o and lse_opt.  Every sample that meets the rank's rows is
 * computed over the parts of the visited blocks inside it, in ring order:
 * bf16 samples eight to a launch (a sample spanning more than eight visited
 * blocks in a launch of its own), fp32 samples one launch each.
 * RA_ERR_SHAPE for boundaries that do not increase from 0 or
 * end past P*Sb; otherwise as ra_ring_attn_fwd. */
ra_status ra_ring_attn_fwd_varlen(const void* q_r, const void* const* k_blocks,
                                  const void* const* v_blocks, int Sb, int H, int D,
                                  int P, int rank, ra_dtype dt, float scale, int causal,
                                  const long long* cu_seqlens, int n_seqs, void* o,
                                  float* lse_opt, void* stream);

/* The whole ring of rank `rank` over zigzag shares in one launch ([RA]
 * §3.2-§3.4 with the sharding of ra_zigzag_schedule).  q_r [B,Sr,H,D] is
 * the rank's share: rows [0, Sr/2) are chunk rank (global rows
 * rank*Sr/2 ..), rows [Sr/2, Sr) chunk 2P-1-rank.  k_shares[j], v_shares[j]
 * ([B,Sr,H,D] each, HOST arrays of P device pointers) are rank j's shares
 * laid out the same way.  Shares are visited in the order (rank - t) mod P;
 * chunks in the future of every query of the share (causal) are never
 * read.  Output o [B,Sr,H,D] in dt for the rank's rows in share order,
 * lse_opt [B,Sr,H] fp32 natural log-sum-exp (may be NULL).  valid_len: real
 * global length (< 0 means P*Sr).  Sr must be a multiple of 128
 * (RA_ERR_SHAPE otherwise; pad to ra_zigzag_padded_len).  P at most
 * RA_MAX_P/2 (RA_ERR_RANGE).  Other errors as ra_ring_attn_fwd. */
ra_status ra_zigzag_attn_fwd(const void* q_r, const void* const* k_shares,
                             const void* const* v_shares, int B, int Sr, int H,
                             int D, int P, int rank, ra_dtype dt, float scale,
                             int causal, long long valid_len, void* o,
                             float* lse_opt, void* stream);

/* Backward of one round ([RA] §3.3 closing paragraph, §6.2): the gradient
 * terms of one K/V block for one query shard, the unit the ring backward
 * repeats as each block arrives.  q, o (the forward's final output), dout
 * [B,Sq,H,D] and k, v [B,Sk,H,D]: device, all bf16 or all fp32, contiguous; lse [B,Sq,H]
 * fp32, the natural log-sum-exp of the WHOLE forward (over every block the
 * rows attend to, as ra_ring_attn_fwd returns it), so that
 * P = exp(scale * Q K^T - lse) are this block's true probabilities
 * (masked pairs 0).  Global positions q_pos0 / k_pos0, causal and
 * valid_len (< 0: no padding) as in ra_block_attn_fwd.  With
 * D = rowsum(dO * O), accumulates (+=, the caller zeroes):
 *   dq [B,Sq,H,D] fp32 += scale * (P * (dO V^T - D)) K
 *   dk [B,Sk,H,D] fp32 += scale * (P * (dO V^T - D))^T Q
 *   dv [B,Sk,H,D] fp32 += P^T dO
 * A block with no visible pair (SKIP) returns at once without touching
 * anything.  stats_ws: fp32 scratch of 2*B*Sq*H floats the call
 * overwrites.  Two launches on `stream`.  bf16 inputs round P and dS to
 * bf16 before their products (as the forward rounds P); fp32 inputs round
 * nothing (a plain kernel pair, the fp32 tier).  D 64 or 128; tensors
 * 16-byte aligned
 * (RA_ERR_SHAPE); NULL pointers with non-empty sizes RA_ERR_NULL. */
ra_status ra_block_attn_bwd(const void* q, const void* k, const void* v,
                            const void* o, const void* dout, const float* lse,
                            int B, int Sq, int Sk, int H, int D, ra_dtype dt,
                            float scale, long long q_pos0, long long k_pos0,
                            int causal, long long valid_len, float* dq,
                            float* dk, float* dv, float* stats_ws,
                            void* stream);

/* Backward of rank `rank`'s ring ([RA] §3.3 closing paragraph, §6.2): the
 * gradients of the loss with respect to the rank's queries and to the K/V
 * blocks it visits, given the upstream gradient dO.  Inputs (device, bf16 or fp32,
 * [B,Sb,H,D] contiguous): q_r, o_r (the forward's output), do_r; lse_r
 * [B,Sb,H] fp32 natural log-sum-exp of the forward (ra_ring_attn_fwd's
 * lse).  k_blocks / v_blocks as in ra_ring_attn_fwd.  With P_j =
 * exp(scale * Q_r K_j^T - lse_r) over the visible pairs of block j (the
 * forward's probabilities, recomputed) and D = rowsum(dO * O):
 *   dq_r          += scale * sum_j (P_j * (dO V_j^T - D)) K_j
 *   dk_blocks[j]  += scale * (P_j * (dO V_j^T - D))^T Q_r
 *   dv_blocks[j]  += P_j^T dO
 * Padding queries (global position >= valid_len) are discarded outputs,
 * not part of the loss: their rows of P are taken as zero, so whatever
 * do_r holds there reaches no gradient and their dq rows get nothing.
 * All three are fp32 [B,Sb,H,D] device buffers, ACCUMULATED into (the
 * caller zeroes them; summing dk/dv over all ranks' calls gives the owners'
 * gradients, as the ring returns them).  dk_blocks / dv_blocks are HOST
 * arrays of P device pointers; entries of blocks the rank skips (causal
 * future) may be NULL and are not touched.  stats_ws: fp32 scratch of
 * 2*B*Sb*H floats the call overwrites (per-row base-2 lse and -D, [2,B,H,Sb]).
 * Two launches on `stream` (dq and the row statistics, then dk/dv).
 * bf16 or fp32 inputs, as in ra_block_attn_bwd.  Errors as
 * ra_ring_attn_fwd. */
ra_status ra_ring_attn_bwd(const void* q_r, const void* const* k_blocks,
                           const void* const* v_blocks, const void* o_r,
                           const void* do_r, const float* lse_r, int B, int Sb,
                           int H, int D, int P, int rank, ra_dtype dt, float scale,
                           int causal, long long valid_len, float* dq_r,
                           float* const* dk_blocks, float* const* dv_blocks,
                           float* stats_ws, void* stream);

/* Grouped-query form of ra_ring_attn_bwd ([RA] §3.5 and §6 name GQA): q_r,
 * o_r, do_r, dq_r [B,Sb,H,D]; every k_blocks[j] / v_blocks[j] and
 * dk_blocks[j] / dv_blocks[j] [B,Sb,H_kv,D] (bf16 / fp32).  Query head h
 * uses K/V head h / (H / H_kv), so the dK/dV of a K/V head sum the terms of
 * its H / H_kv query heads.  RA_ERR_SHAPE unless H_kv > 0 divides H;
 * everything else as ra_ring_attn_bwd. */
ra_status ra_ring_attn_bwd_gqa(const void* q_r, const void* const* k_blocks,
                               const void* const* v_blocks, const void* o_r,
                               const void* do_r, const float* lse_r, int B, int Sb,
                               int H, int H_kv, int D, int P, int rank, ra_dtype dt,
                               float scale, int causal, long long valid_len,
                               float* dq_r, float* const* dk_blocks,
                               float* const* dv_blocks, float* stats_ws, void* stream);

/* Backward over packed samples (the form of ra_ring_attn_fwd_varlen): B =
 * 1, sample i holds global positions [cu_seqlens[i], cu_seqlens[i+1]) and
 * its rows attend only within it ([RA] §6).  q_r, o_r, do_r [1,Sb,H,D] bf16 or fp32,
 * lse_r [1,Sb,H] (ra_ring_attn_fwd_varlen's lse); k_blocks / v_blocks and
 * dk_blocks / dv_blocks as in ra_ring_attn_bwd.  Accumulates (+=) dq_r and
 * the dK/dV parts of the visited blocks; rows outside every sample are not
 * touched.  One launch pair per sample that meets the rank's rows, over the
 * parts of the visited blocks inside that sample.  stats_ws: fp32 scratch
 * of 2*Sb*H floats.  Errors as ra_ring_attn_fwd_varlen and
 * ra_ring_attn_bwd. */
ra_status ra_ring_attn_bwd_varlen(const void* q_r, const void* const* k_blocks,
                                  const void* const* v_blocks, const void* o_r,
                                  const void* do_r, const float* lse_r, int Sb, int H,
                                  int D, int P, int rank, ra_dtype dt, float scale,
                                  int causal, const long long* cu_seqlens, int n_seqs,
                                  float* dq_r, float* const* dk_blocks,
                                  float* const* dv_blocks, float* stats_ws, void* stream);

/* Backward of rank `rank`'s zigzag ring ([RA] §3.4 load balancing with
 * the backward of §3.3 closing paragraph, §6.2): as ra_ring_attn_bwd over
 * the shares of ra_zigzag_attn_fwd.  q_r, o_r, do_r [B,Sr,H,D] bf16 or fp32 (chunk
 * rank then chunk 2P-1-rank), lse_r [B,Sr,H] fp32 (ra_zigzag_attn_fwd's
 * lse); k_shares / v_shares HOST arrays of P device pointers to every
 * rank's [B,Sr,H,D] share.  Accumulates (+=) dq_r [B,Sr,H,D] fp32 and, into
 * dk_shares[j] / dv_shares[j] (fp32 [B,Sr,H,D], entries of shares the rank
 * skips may be NULL), the parts of share j's two chunks; summed over all
 * ranks they are the owners' gradients.  stats_ws: fp32 scratch of
 * 2*B*Sr*H floats.  Sr a multiple of 128, P at most RA_MAX_P/2, bf16 or
 * fp32 inputs; other errors as ra_ring_attn_bwd.  Two launches on `stream`. */
ra_status ra_zigzag_attn_bwd(const void* q_r, const void* const* k_shares,
                             const void* const* v_shares, const void* o_r,
                             const void* do_r, const float* lse_r, int B, int Sr,
                             int H, int D, int P, int rank, ra_dtype dt, float scale,
                             int causal, long long valid_len, float* dq_r,
                             float* const* dk_shares, float* const* dv_shares,
                             float* stats_ws, void* stream);

/* Ulysses sequence-shard -> head-shard transpose ([RA] §3.5) of the P
 * per-rank tensors stacked rank-major:
 *   src [P, B, S/P, H, D]  ->  dst [P, B, S, H/P, D]
 *   dst[r, b, j*S/P + s, h', d] = src[j, b, s, r*H/P + h', d]
 * S is the GLOBAL length.  A pure bit copy of elem_bytes-sized elements
 * (1, 2, 4 or 8), bit-exact for any payload (NaN, -0).  src and dst must not
 * overlap.  Errors: RA_ERR_NULL, RA_ERR_SHAPE (S % P or H % P non-zero,
 * [UG] §三), RA_ERR_DTYPE (elem_bytes), RA_ERR_HIP. */
ra_status ra_seq2head(const void* src, void* dst, int P, int B, long long S,
                      int H, int D, int elem_bytes, void* stream);

/* The inverse: src [P, B, S, H/P, D] -> dst [P, B, S/P, H, D]
 *   dst[j, b, s, r*H/P + h', d] = src[r, b, j*S/P + s, h', d]
 * Same arguments and errors as ra_seq2head. */
ra_status ra_head2seq(const void* src, void* dst, int P, int B, long long S,
                      int H, int D, int elem_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
