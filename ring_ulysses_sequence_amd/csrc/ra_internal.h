// Internal declarations shared by the host-side translation units of
// libringattn.so: the thread-local error state and the host schedule helpers.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "ringattn.h"

namespace ra {

// Record an error message for ra_last_error() and return `st`.
ra_status fail(ra_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

// Clear the thread's error message (every entry point starts with this).
void clear_error();

// Class of query positions [q0, q1) against key positions [k0, k1)
// ([RA] §3.4): range comparisons on global positions, keys >= valid_len
// being padding.  `valid_len` must already be normalised (>= 0).
int block_class(long long q0, long long q1, long long k0, long long k1,
                bool causal, long long valid_len);

// Workgroup slots of the chip for the 128-row attention kernels: two per
// compute unit (their LDS use) on 256 compute units.
constexpr long long kWorkgroupSlots = 512;

// The merge of a split ring: output row (b, r, h) of the [B, Sq, H, D]
// output combines row r % 128 of slots ((b*H + h)*ceil(Sq/128) + r/128)*nsplit
// + j, j < nsplit, each a normalised fp32 partial o ([slot][128][D]) with its
// natural lse ([slot][128]).  o is written in bf16 (out_bf16) or fp32, lse
// when not NULL.
struct SplitMergeArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int B, Sq, H, D;
  int nsplit, out_bf16;
};
ra_status merge_split(const char* name, const SplitMergeArgs& m, void* stream);

// Current value of a process-wide option (see ra_set_option).
int option(int which);

}  // namespace ra
