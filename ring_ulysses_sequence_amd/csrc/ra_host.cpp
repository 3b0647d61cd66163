// Host-only part of libringattn.so: error state, padding and shard cover,
// ring order and block classification.  No HIP calls; also builds with a
// plain host compiler.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <string>

#include "ra_internal.h"

namespace ra {

static thread_local std::string g_last_error;

ra_status fail(ra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

static std::atomic<int> g_options[RA_OPT_COUNT];

int option(int which) {
  return (which >= 0 && which < RA_OPT_COUNT) ? g_options[which].load(std::memory_order_relaxed) : 0;
}

// The three cases of [RA] §3.4 as range comparisons.  With K the set of
// real keys [k0, min(k1, valid_len)):
//   no real key, or (causal) the first key after the last query -> SKIP;
//   all keys real and (non-causal, or the last key at or before the first
//   query)                                                      -> FULL;
//   otherwise some but not all pairs are visible                -> DIAG.
int block_class(long long q0, long long q1, long long k0, long long k1,
                bool causal, long long valid_len) {
  if (q1 <= q0 || k1 <= k0) return RA_SKIP;
  if (k0 >= valid_len) return RA_SKIP;
  if (causal && k0 > q1 - 1) return RA_SKIP;
  const bool all_real = k1 <= valid_len;
  if (all_real && (!causal || k1 - 1 <= q0)) return RA_FULL;
  return RA_DIAG;
}

}  // namespace ra

extern "C" {

int ra_abi_version(void) { return 2; }

ra_status ra_set_option(int opt, int value) {
  ra::clear_error();
  if (opt == RA_OPT_ATTN_KERNEL) {
    if (value != RA_KERNEL_AUTO && value != RA_KERNEL_ROWMAX)
      return ra::fail(RA_ERR_RANGE, "ra_set_option: unknown kernel choice %d", value);
    ra::g_options[opt].store(value, std::memory_order_relaxed);
    return RA_OK;
  }
  if (opt == RA_OPT_ATTN_WAVES) {
    if (value != 0 && value != 4 && value != 8)
      return ra::fail(RA_ERR_RANGE, "ra_set_option: waves per workgroup must be 0, 4 or 8 "
                      "(got %d)", value);
    ra::g_options[opt].store(value, std::memory_order_relaxed);
    return RA_OK;
  }
  return ra::fail(RA_ERR_RANGE, "ra_set_option: unknown option %d", opt);
}

int ra_get_option(int opt) { return ra::option(opt); }

const char* ra_last_error(void) { return ra::g_last_error.c_str(); }

long long ra_padded_len(long long S, int P, int pad_multiple) {
  ra::clear_error();
  if (S < 0 || P <= 0 || pad_multiple <= 0) {
    ra::fail(RA_ERR_SHAPE, "ra_padded_len: need S >= 0, P > 0, pad_multiple > 0 "
             "(got S=%lld P=%d pad_multiple=%d)", S, P, pad_multiple);
    return -1;
  }
  const long long unit = (long long)P * pad_multiple;
  return (S + unit - 1) / unit * unit;
}

ra_status ra_shard_range(long long S, int P, int rank, long long* begin,
                         long long* end) {
  ra::clear_error();
  if (!begin || !end) return ra::fail(RA_ERR_NULL, "ra_shard_range: NULL output");
  if (P <= 0 || S < 0)
    return ra::fail(RA_ERR_SHAPE, "ra_shard_range: need P > 0 and S >= 0");
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "ra_shard_range: rank %d outside [0, %d)", rank, P);
  if (S % P != 0) {
    const long long unit = (long long)P * RA_PAD_MULTIPLE;
    return ra::fail(RA_ERR_SHAPE,
                    "sequence length %lld is not divisible by P=%d; pad it to "
                    "%lld (ra_padded_len)", S, P, (S + unit - 1) / unit * unit);
  }
  const long long per = S / P;
  *begin = rank * per;
  *end = (rank + 1) * per;
  return RA_OK;
}

ra_status ra_classify_block(long long q0, long long q1, long long k0,
                            long long k1, int causal, long long valid_len,
                            int* cls) {
  ra::clear_error();
  if (!cls) return ra::fail(RA_ERR_NULL, "ra_classify_block: NULL output");
  if (valid_len < 0) valid_len = INT64_MAX;
  *cls = ra::block_class(q0, q1, k0, k1, causal != 0, valid_len);
  return RA_OK;
}

ra_status ra_ring_schedule(int P, int rank, long long block_len, int causal,
                           long long valid_len, int* src_out, int* class_out) {
  ra::clear_error();
  if (!src_out || !class_out)
    return ra::fail(RA_ERR_NULL, "ra_ring_schedule: NULL output array");
  if (P <= 0 || block_len < 0)
    return ra::fail(RA_ERR_SHAPE, "ra_ring_schedule: need P > 0 and block_len >= 0");
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "ra_ring_schedule: rank %d outside [0, %d)", rank, P);
  if (valid_len < 0) valid_len = (long long)P * block_len;
  const long long q0 = rank * block_len, q1 = q0 + block_len;
  for (int t = 0; t < P; ++t) {
    const int j = ((rank - t) % P + P) % P;  // [RA] §3.3
    src_out[t] = j;
    class_out[t] = ra::block_class(q0, q1, j * block_len, (j + 1) * block_len,
                                   causal != 0, valid_len);
  }
  return RA_OK;
}

long long ra_zigzag_padded_len(long long S, int P) {
  ra::clear_error();
  if (S < 0 || P <= 0) {
    ra::fail(RA_ERR_SHAPE, "ra_zigzag_padded_len: need S >= 0 and P > 0 (got S=%lld P=%d)",
             S, P);
    return -1;
  }
  const long long unit = 2LL * P * 64;  // 2P chunks of a multiple of 64 rows
  return (S + unit - 1) / unit * unit;
}

ra_status ra_zigzag_schedule(int P, int rank, long long chunk_len, int causal,
                             long long valid_len, int* src_out, int* class_out) {
  ra::clear_error();
  if (!src_out || !class_out)
    return ra::fail(RA_ERR_NULL, "ra_zigzag_schedule: NULL output array");
  if (P <= 0 || chunk_len < 0)
    return ra::fail(RA_ERR_SHAPE, "ra_zigzag_schedule: need P > 0 and chunk_len >= 0");
  if (rank < 0 || rank >= P)
    return ra::fail(RA_ERR_RANGE, "ra_zigzag_schedule: rank %d outside [0, %d)", rank, P);
  if (valid_len < 0) valid_len = 2LL * P * chunk_len;
  // the query share: chunk rank and chunk 2P-1-rank, positions increasing;
  // a key chunk is classified against [first query, last query] (SKIP only
  // if it is in the future of both query chunks, FULL only if it is in the
  // past of both), which is what the kernel needs: within a DIAG chunk each
  // wave still decides per tile on its own rows
  const long long q0 = rank * chunk_len;
  const long long q1 = (2LL * P - 1 - rank) * chunk_len + chunk_len;
  for (int t = 0; t < P; ++t) {
    const int j = ((rank - t) % P + P) % P;  // [RA] §3.3
    src_out[t] = j;
    for (int half = 0; half < 2; ++half) {
      const long long kc = half == 0 ? j : 2LL * P - 1 - j;
      class_out[2 * t + half] = ra::block_class(q0, q1, kc * chunk_len, (kc + 1) * chunk_len,
                                                causal != 0, valid_len);
    }
  }
  return RA_OK;
}

}  // extern "C"
