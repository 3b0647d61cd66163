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

// Launch the n-way merge of split-ring partials (o_part [nsplit, rows, D]
// fp32, lse_part [nsplit, rows]) into o (rows x D in dt) and lse_opt.
ra_status merge_splits(const char* name, const float* o_part, const float* lse_part, int nsplit,
                       long long rows, int D, void* o, ra_dtype dt, float* lse_opt,
                       void* stream);

// Slices worth splitting a ring's visited blocks into (1: none), from the
// grid of 128-row workgroups against the chip's workgroup slots.
int split_hint(long long base_workgroups, int visited);

// Current value of a process-wide option (see ra_set_option).
int option(int which);

}  // namespace ra
