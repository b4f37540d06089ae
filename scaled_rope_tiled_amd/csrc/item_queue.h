// Run-time assignment of work items to the workgroups of the tiled attention
// kernels (a scheduling block of kSchedWords zero-filled 64-bit counters).
#pragma once
#include <hip/hip_runtime.h>

#include "srt_internal.h"

namespace srt {

// Run-time assignment of (head, tile) work items to workgroups.
//
// Items are numbered heavy first: item = (y * B + b) * HX + x, with x the
// workgroup head (HX of them), b the batch and y the tile rank (y = 0 is the
// tile with the most work under the causal mask: the last query tile of the
// forward and dq kernels, the first key block of the dk/dv kernel).  The
// hardware hands workgroups to the eight XCDs in turn, so every XCD runs the
// same number of them, and with a fixed assignment (item =
// workgroup index) XCD k runs heads x = k mod 8: its L2 keeps their K/V, but
// XCDs that run slower (measured: up to 3 % on one chip) finish last.  With a
// scheduling block each workgroup instead takes the next item from
//   1. its own XCD's queue: the heads x = k mod 8, tiles y < ysplit;
//   2. once that is empty, one shared pool: every head, the light tail
//      y >= ysplit (the last quarter of the tiles), heavy first;
//   3. then any other XCD's queue (there are as many items as workgroups, so
//      a workgroup always finds one, whatever the hardware's distribution).
// A faster XCD reaches the pool sooner and takes its heavier items, which
// evens out the finishing times while the heavy items keep their locality.
// Each queue is a counter in the block: atomicAdd hands out index old and the
// item exists while old < the queue's length.
__device__ inline int sched_take(unsigned long long* blk, int HX, int B, int ntq) {
  const int ysplit = ntq - (ntq >= 4 ? ntq / 4 : 0);
  const int own = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7);   // this XCD
  for (int t = 0; t < 9; ++t) {
    if (t == 1) {
      const long long n = (long long)(ntq - ysplit) * B * HX;
      if (n == 0) continue;
      const long long idx = (long long)atomicAdd(&blk[8], 1ull);
      if (idx < n) {
        const int per_y = B * HX;
        const int yy = ysplit + (int)(idx / per_y), r = (int)(idx % per_y);
        return (yy * B + r / HX) * HX + r % HX;
      }
      continue;
    }
    const int k = t == 0 ? own : (own + t - 1) & 7;   // t = 2..8: the other seven queues
    const int nh = k < HX ? (HX - 1 - k) / 8 + 1 : 0;   // heads k, k + 8, ... below HX
    const long long n = (long long)nh * B * ysplit;
    if (n == 0) continue;
    const long long idx = (long long)atomicAdd(&blk[k], 1ull);
    if (idx < n) {
      const int per_y = nh * B;
      const int yy = (int)(idx / per_y), r = (int)(idx % per_y);
      const int bb = r / nh;
      return (yy * B + bb) * HX + k + 8 * (r - bb * nh);
    }
  }
  return 0;   // not reached from a zero-filled block
}

// The launch's last workgroup zero-fills the block again for the next call.
__device__ inline void sched_release(unsigned long long* blk, unsigned nwg) {
  if (atomicAdd(&blk[9], 1ull) == (unsigned long long)nwg - 1) {
    for (int k = 0; k < kSchedWords; ++k) atomicExch(&blk[k], 0ull);
  }
}

}  // namespace srt
