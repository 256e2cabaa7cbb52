// Input side of the prepare-style kernels (MXFP4 and NVFP4 prepare, the
// weight quantisers): which 32-entry block of which row a lane owns, and the
// bf16 loads of a block.
#pragma once

#include "sharq_device.h"

namespace sharq {

// Lane -> (row, block) map shared by the prepare and quantise kernels. A wave
// owns a band of 16 rows and one 128-entry K stage (4 blocks): lane l takes
// row 16 * band + l / 4 and block 4 * stage + l % 4. In the stage-major
// layout its codes are then one contiguous 1 KB run per code array and its
// scales one 64-byte run; each row's input is read in 256-byte runs.
struct BlockOfLane {
  uint32_t t, b;
  bool row_ok, block_ok;
};

__device__ __forceinline__ BlockOfLane block_of_item(uint32_t item, uint32_t lane, uint32_t stages,
                                                     uint32_t blocks_per_row, uint32_t rows) {
  const uint32_t band = item / stages;
  const uint32_t g = item - band * stages;
  BlockOfLane r;
  r.t = band * 16 + (lane >> 2);
  r.b = g * 4 + (lane & 3);
  r.row_ok = r.t < rows;
  r.block_ok = r.row_ok && r.b < blocks_per_row;
  return r;
}
__device__ __forceinline__ BlockOfLane block_of_lane(uint32_t stages, uint32_t blocks_per_row, uint32_t rows) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  return block_of_item(gid >> 6, gid & 63, stages, blocks_per_row, rows);
}



__device__ __forceinline__ void load_block(const uint16_t* p, uint4 (&raw)[4]) {
  const uint4* src = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src[i];
}

__device__ __forceinline__ void widen_block(const uint4 (&raw)[4], float (&xv)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] = bf16_lo(w[j]);
      xv[8 * i + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
}

__device__ __forceinline__ void times_gamma(float (&xv)[32], const uint4 (&graw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {graw[i].x, graw[i].y, graw[i].z, graw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] *= bf16_lo(w[j]);
      xv[8 * i + 2 * j + 1] *= bf16_hi(w[j]);
    }
  }
}

}  // namespace sharq
