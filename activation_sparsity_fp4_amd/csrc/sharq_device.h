// Device-side building blocks shared by the SharQ kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// MX block length along K (one E8M0 scale per 32 consecutive entries).
constexpr int kBlock = 32;

// bf16 bit pattern -> float (exact). A dword holds two bf16: low half = even index.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats rounded to bf16 (nearest, ties to even) by one gfx950
// v_cvt_pk_bf16_f32: the low half holds a, the high half b. Finite inputs
// (fp32 denormals are kept, so they round like every other value).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// E8M0 byte (exponent + 127) of a block from the bit pattern of its largest
// magnitude (sign bit clear): floor(log2(amax)) - 2, clamped below at -127.
// For a normal amax with exponent field f this is f - 129 (byte f - 2); f < 2
// (amax < 2^-125, including subnormals and zero) clamps to byte 0. The upper
// clamp never triggers for finite inputs (f <= 254 gives byte 252).
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  uint32_t f = amax_bits >> 23;
  return f > 2u ? f - 2u : 0u;
}

// 2^(byte - 127) as a float; byte 0 is the subnormal 2^-127.
__device__ __forceinline__ float scale_from_e8m0(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

// 32 floats -> 16 bytes of E2M1 codes, x / scale rounded to nearest-even and
// saturated at 6 by the gfx950 scaled converter (sign kept on zero results).
__device__ __forceinline__ uint4 quantize32(const float (&v)[32], float scale) {
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 0], v[8 * d + 1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 2], v[8 * d + 3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 4], v[8 * d + 5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 6], v[8 * d + 7], scale, 3);
    w[d] = r;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16 bytes of E2M1 codes -> 32 floats code * scale (exact).
__device__ __forceinline__ void dequantize32(uint4 c, float scale, float (&q)[32]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], scale, 0);
    v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], scale, 1);
    v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], scale, 2);
    v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], scale, 3);
    q[8 * d + 0] = p0[0]; q[8 * d + 1] = p0[1];
    q[8 * d + 2] = p1[0]; q[8 * d + 3] = p1[1];
    q[8 * d + 4] = p2[0]; q[8 * d + 5] = p2[1];
    q[8 * d + 6] = p3[0]; q[8 * d + 7] = p3[1];
  }
}

// Layout shared by every kernel: an MXFP4 [rows x K] tensor is stored
// stage-major, grouped by 128-entry K stage (G = ceil(K/128) stages).
//   codes  [G][rows][64]: the 16 code bytes of block b of a row sit at byte
//          16 * (b % 4) of the row's 64-byte chunk in stage b / 4;
//   scales [G][rows][4]:  the E8M0 byte of block b is byte b % 4 of the row's
//          dword in stage b / 4.
// One GEMM stage of a row tile is then one contiguous run of codes and one of
// scales, so its loads use whole cache lines. Blocks of a last, partial stage
// past K / 32 have zero codes and zero scale bytes.
__device__ __forceinline__ int64_t scale_index(int64_t row, uint32_t block, int64_t rows) {
  return (int64_t)(block >> 2) * rows * 4 + row * 4 + (block & 3);
}
__device__ __forceinline__ int64_t code_offset(int64_t row, uint32_t block, int64_t rows) {
  return (int64_t)(block >> 2) * rows * 64 + row * 64 + (block & 3) * 16;
}

// Largest |v| of 32 finite floats as a bit pattern (sign cleared). A float
// max of magnitudes (abs is a free input modifier, three inputs per
// instruction) returns exactly the largest magnitude; if denormals were
// flushed only blocks whose largest magnitude is subnormal could differ, and
// those get scale byte 0 either way.
__device__ __forceinline__ uint32_t amax_bits32(const float (&v)[32]) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) m = fmaxf(m, fabsf(v[k]));
  return __float_as_uint(m);
}

}  // namespace sharq
