// CDNA4 (gfx950) building blocks for kernels that copy tiles HBM -> LDS with
// the buffer unit (buffer_load ... lds) while reading other LDS buffers:
// buffer descriptors, explicit wait counters, and LDS operand reads that the
// compiler's wait insertion does not see.
//
// Why the reads are inline assembly: the compiler cannot tell which LDS bytes
// an LDS-DMA copy writes, so before every LDS read it can see it waits for all
// copies in flight, which would serialise each tile's copy with the compute
// that is meant to hide it.  A read made here is invisible to that analysis;
// its result must be claimed with claim_lds<N> before use, and the copies it
// must not overtake are ordered by the caller's explicit waits and barriers.
#pragma once

#include <hip/hip_runtime.h>

namespace ra_cdna4 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Word 3 of a raw (untyped, unswizzled) buffer descriptor.
constexpr int kRsrcWord3 = 0x00020000;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(lds_void_ptr)p;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ds_read_b128 / ds_read_b64_tr_b16 at LDS byte address addr + OFF.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// ds_write_b128 of v at LDS byte address addr + OFF (complete once lgkmcnt
// has counted it out, e.g. at pipeline_barrier).
template <int OFF>
__device__ __forceinline__ void lds_write_b128(unsigned addr, u32x4 v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "n"(OFF));
}

// Wait until at most N LDS (or scalar-memory) operations of this wave are
// outstanding, and make `x` depend on the wait so that no use of it is
// scheduled before.  LDS operations complete in issue order, so with N = the
// number of LDS reads issued after the one that produced x, x is ready.
template <int N, typename T>
__device__ __forceinline__ void claim_lds(T& x) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}
// claim_lds with a count that is a constant only after loop unrolling.
template <typename T>
__device__ __forceinline__ void claim_lds_n(int n, T& x) {
  switch (n) {
    case 0: claim_lds<0>(x); break;
    case 1: claim_lds<1>(x); break;
    case 2: claim_lds<2>(x); break;
    case 3: claim_lds<3>(x); break;
    case 4: claim_lds<4>(x); break;
    case 5: claim_lds<5>(x); break;
    case 6: claim_lds<6>(x); break;
    case 7: claim_lds<7>(x); break;
    default: claim_lds<8>(x); break;
  }
}

// Workgroup barrier for a copy pipeline.  The caller has already waited
// (vmcnt) for the copies that must be visible after it.  All of this wave's
// LDS reads have returned (lgkmcnt(0)), so the buffers they read may be
// overwritten once every wave has arrived.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace ra_cdna4
