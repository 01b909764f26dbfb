// Copies of planned blobs from host memory into pool slots, by the CUs over
// PCIe (pinned host memory mapped for the device), for the refills planned
// on the device (moe_layer_forward_offload).
#ifndef MOE355_PULL_H
#define MOE355_PULL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Byte range [off16, off16 + n16) of 16-byte pieces of every planned blob:
// plan = [0] loads, then experts [E], slots [E] (device); blocks = the
// number of blocks that share the copy (0: none).
struct PullJob {
  const uint4* src;
  uint4* dst;
  long src_stride16, dst_stride16, off16, n16;
  const int32_t* plan;
  int E;
  int blocks;
};

// Block b of j.blocks, blob after blob: four pieces per thread in flight
// (named registers, no array: inside a large kernel an array may be left in
// scratch memory), clamped loads and guarded stores.
__device__ __forceinline__ void plan_pull_body(PullJob j, int b) {
  const int nb = j.plan[0];
  const long step = (long)j.blocks * blockDim.x;
  for (int k = 0; k < nb; ++k) {
    const uint4* __restrict__ src = j.src + (long)j.plan[1 + k] * j.src_stride16 + j.off16;
    uint4* __restrict__ dst = j.dst + (long)j.plan[1 + j.E + k] * j.dst_stride16 + j.off16;
    for (long q = (long)b * blockDim.x + threadIdx.x; q < j.n16; q += 4 * step) {
      const long q1 = q + step, q2 = q + 2 * step, q3 = q + 3 * step;
      const uint4 v0 = src[q];
      const uint4 v1 = src[q1 < j.n16 ? q1 : q];
      const uint4 v2 = src[q2 < j.n16 ? q2 : q];
      const uint4 v3 = src[q3 < j.n16 ? q3 : q];
      dst[q] = v0;
      if (q1 < j.n16) dst[q1] = v1;
      if (q2 < j.n16) dst[q2] = v2;
      if (q3 < j.n16) dst[q3] = v3;
    }
  }
}

}  // namespace moe

#endif  // MOE355_PULL_H
