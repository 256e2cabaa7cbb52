// Layout conversion between the canonical row-major block-FP4 layout and the
// stage-major layout every SharQ kernel reads (pure data movement).
//
// Row-major (the layout an external MXFP4 or NVFP4 quantiser writes):
//   codes  [R][K/2]  (two E2M1 codes per byte, even K index in the low nibble),
//   scales [R][K/B]  (one byte per block of B = 32 (E8M0) or 16 (E4M3) entries).
// Stage-major (G = ceil(K/128) stages of 128 entries):
//   codes  [G][R][64],  scales [G][R][128/B];  bytes past K are zero.
// Both directions keep every code and scale byte; packing zero-fills the
// bytes of a last, partial stage past K.

#include "sharq_internal.h"

namespace sharq {
namespace {

// One lane per 16-byte code chunk of the stage-major tensor (G * R * 4 chunks).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ rm, int64_t R, int64_t row_bytes,
                                                         int64_t chunks, uint8_t* __restrict__ sm) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t part = c & 3, r = (c >> 2) % R, g = (c >> 2) / R;
  const int64_t off = 64 * g + 16 * part;  // byte offset inside the row-major row
  const uint4 v = off < row_bytes ? *reinterpret_cast<const uint4*>(rm + r * row_bytes + off) : make_uint4(0, 0, 0, 0);
  reinterpret_cast<uint4*>(sm)[c] = v;
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint8_t* __restrict__ sm, int64_t R,
                                                           int64_t row_bytes, int64_t chunks,
                                                           uint8_t* __restrict__ rm) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t part = c & 3, r = (c >> 2) % R, g = (c >> 2) / R;
  const int64_t off = 64 * g + 16 * part;
  if (off < row_bytes) *reinterpret_cast<uint4*>(rm + r * row_bytes + off) = reinterpret_cast<const uint4*>(sm)[c];
}

// One lane per scale byte of the stage-major tensor (G * R * per_stage bytes).
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ rm, int64_t R,
                                                          int64_t row_bytes, int per_stage, int64_t n,
                                                          uint8_t* __restrict__ sm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t b = i % per_stage, r = (i / per_stage) % R, g = i / per_stage / R;
  const int64_t off = per_stage * g + b;
  sm[i] = off < row_bytes ? rm[r * row_bytes + off] : (uint8_t)0;
}

__global__ __launch_bounds__(256) void unpack_scales_kernel(const uint8_t* __restrict__ sm, int64_t R,
                                                            int64_t row_bytes, int per_stage, int64_t n,
                                                            uint8_t* __restrict__ rm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t b = i % per_stage, r = (i / per_stage) % R, g = i / per_stage / R;
  const int64_t off = per_stage * g + b;
  if (off < row_bytes) rm[r * row_bytes + off] = sm[i];
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes_rm, const uint8_t* scales_rm, int64_t R, int64_t K, int block,
                       uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t G = (K + 127) / 128, chunks = G * R * 4;
  const int per_stage = 128 / block;
  const int64_t n = G * R * per_stage;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, codes_rm, R,
                     K / 2, chunks, codes);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, scales_rm, R,
                     K / block, per_stage, n, scales);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t K, int block,
                         uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t stream) {
  const int64_t G = (K + 127) / 128, chunks = G * R * 4;
  const int per_stage = 128 / block;
  const int64_t n = G * R * per_stage;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, codes, R,
                     K / 2, chunks, codes_rm);
  hipLaunchKernelGGL(unpack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, scales, R,
                     K / block, per_stage, n, scales_rm);
  return hipGetLastError();
}

}  // namespace sharq
