// Calibration kernel for the GEMM roofline: the FP4 scaled-MFMA rate this GPU
// sustains on register operands, with no memory traffic at all. The published
// dense FP4 peak assumes the top clock; with realistic (random) operands the
// matrix cores draw enough power that the clock drops, so the rate a kernel
// can reach is lower. The benchmark reports this figure beside the published
// peak (and the same for the fp16 MFMA). Not part of the SharQ library: it is
// built as its own shared object.
//
// Each wave issues chains of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP4 x FP4) on
// operands filled from a per-lane hash (random bit patterns, so every
// nibble decodes to some E2M1 value), into 8 independent accumulators so that
// no MFMA waits on the one before it. The accumulators are folded into one
// value per wave at the end so that nothing is dead code.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iterations, uint32_t seed, float* __restrict__ out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)mix(seed ^ (gid * 16 + i));
    b[i] = (int)mix(seed ^ (gid * 16 + 8 + i) ^ 0x9e3779b9u);
  }
  const int sa = 127 + (int)(mix(gid) & 3), sb = 127 - (int)(mix(gid + 1) & 3);  // E8M0 near 1
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v16f{};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, sa, 0, sb);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if ((threadIdx.x & 63) == 0) out[gid >> 6] = s;
}

// The same for V_MFMA_F32_32X32X16_F16 (the unit the NVFP4 GEMM runs on):
// random fp16 operands with exponents kept near 1 so no product overflows.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256) void mfma_rate_f16_kernel(int iterations, uint32_t seed, float* __restrict__ out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  v8h a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ra = mix(seed ^ (gid * 16 + i)), rb = mix(seed ^ (gid * 16 + 8 + i) ^ 0x9e3779b9u);
    // sign and 10 mantissa bits random, exponent field 14 or 15 (values in [0.5, 2))
    a[i] = __builtin_bit_cast(_Float16, (uint16_t)((ra & 0x83FFu) | ((14u + ((ra >> 16) & 1u)) << 10)));
    b[i] = __builtin_bit_cast(_Float16, (uint16_t)((rb & 0x83FFu) | ((14u + ((rb >> 16) & 1u)) << 10)));
  }
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v16f{};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if ((threadIdx.x & 63) == 0) out[gid >> 6] = s;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int sharq_calib_mfma_f16(int blocks, int iterations,
                                                                             float* out, hipStream_t stream) {
  if (blocks <= 0 || iterations <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_rate_f16_kernel, dim3(blocks), dim3(256), 0, stream, iterations, 0x1234567u, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" __attribute__((visibility("default"))) int sharq_calib_mfma_fp4(int blocks, int iterations,
                                                                             float* out, hipStream_t stream) {
  if (blocks <= 0 || iterations <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, stream, iterations, 0x1234567u, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
