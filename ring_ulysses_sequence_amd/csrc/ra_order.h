// Workgroup orders shared by the kernels whose workgroups stream K/V tiles
// for a query tile (the forward and the dQ kernel of the backward).
#pragma once

#include <hip/hip_runtime.h>

namespace ra_order {

// Lockstep order for kernels with one workgroup of 256 query rows per CU
// (32 CUs per XCD; workgroups are dispatched round-robin over the 8 XCDs).
// Each XCD takes whole (batch, head) problems, one at a time, so its 32
// resident workgroups share one head's K/V stream in that XCD's L2 -- if
// they walk it at the same time.  A head's Q query tiles (a multiple of 64)
// are taken in pairs of 32-tile chunks from the top:
//   - the later chunk starts together and visits the blocks that every one
//     of its queries sees whole first and the diagonal block last (the
//     caller's rotation `later_rot` of its block table: 1 for a ring share,
//     whose table starts with its own, diagonal block; 2 for a zigzag share,
//     whose table starts with its two own chunks): all 32 stream the full
//     blocks in step, then the diagonal block from its first tile, and tile
//     t of the chunk finishes a fixed number of key tiles after tile t-1;
//   - the earlier chunk is dispatched in decreasing tile order, so its
//     workgroups land on the CUs as the later chunk's finish, and visits the
//     diagonal block first (table order, rot = 0): a workgroup that starts
//     later has that many fewer diagonal tiles, so all of them reach the
//     full blocks at the same step and finish together, and the next head
//     starts in step again.
// id: the workgroup's dispatch index of n (n % 8 == 0, BH % 8 == 0).
// Returns false, and the caller takes its plain order, when the grid does not
// hold whole heads per XCD and whole chunk pairs per head.
__host__ __device__ __forceinline__ bool lockstep_coords(int id, int n, int Q, int BH,
                                                         int later_rot, int& bh, int& qt,
                                                         int& rot) {
  if ((n & 7) != 0 || (Q & 63) != 0 || (BH & 7) != 0) return false;
  const int j = (id & 7) * (n >> 3) + (id >> 3);
  bh = j / Q;
  const int r = j % Q;
  const int top = Q - 64 * (r >> 6), pos = r & 31;
  if (r & 32) {
    qt = top - 33 - pos;
    rot = 0;
  } else {
    qt = top - 32 + pos;
    rot = later_rot;
  }
  return true;
}

}  // namespace ra_order
