// SiLU-gated product between a fused gate|up projection and the down
// projection (glue around the SharQ linears, not part of the method):
// h[t][i] = bf16_rne(silu(g) * u), g = gu[t][i], u = gu[t][I + i].
// HBM-bound elementwise kernel: each lane reads 8 gate and 8 up floats
// (2 x 32 B) and writes 8 bf16 (16 B).

#include "sharq_internal.h"
#include "silu.h"

namespace sharq {
namespace {

__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ gu, int64_t I, uint32_t groups_per_row,
                                                       uint32_t total, uint16_t* __restrict__ h) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const uint32_t t = gid / groups_per_row;
  const uint32_t c = gid - t * groups_per_row;
  const float4* g = reinterpret_cast<const float4*>(gu + (int64_t)t * 2 * I + 8 * (int64_t)c);
  const float4* u = reinterpret_cast<const float4*>(gu + (int64_t)t * 2 * I + I + 8 * (int64_t)c);
  const float4 g0 = g[0], g1 = g[1], u0 = u[0], u1 = u[1];
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = silu_times(gv[2 * k], uv[2 * k]);
    const float b = silu_times(gv[2 * k + 1], uv[2 * k + 1]);
    out[k] = bf16x2_rne(a, b);
  }
  reinterpret_cast<uint4*>(h + (int64_t)t * I)[c] = make_uint4(out[0], out[1], out[2], out[3]);
}

// Weighted combine of a mixture-of-experts layer (glue, not the method):
// out[t][c] = sum over slots j = 0, 1, ..., k-1 of weights[t][j] *
// y[pair_index[t][j]][c] (slots with index -1 skipped), accumulated in fp32
// in slot order with one fused multiply-add per slot, so the result does not
// depend on timing. A lane owns 4 columns of one token row: HBM-bound, k
// gathered 16-byte reads and one 16-byte (fp32) or 8-byte (bf16) write.
__device__ __forceinline__ void combine_store(float4 acc, int64_t t, uint32_t c, int64_t H, float* __restrict__ out,
                                              uint16_t* __restrict__ out_bf16) {
  if (out) reinterpret_cast<float4*>(out + t * H)[c] = acc;
  if (out_bf16) {
    const uint32_t lo = bf16x2_rne(acc.x, acc.y);
    const uint32_t hi = bf16x2_rne(acc.z, acc.w);
    reinterpret_cast<uint2*>(out_bf16 + t * H)[c] = make_uint2(lo, hi);
  }
}

__device__ __forceinline__ void combine_fma(float4& acc, float w, float4 v) {
  acc.x = fmaf(w, v.x, acc.x);
  acc.y = fmaf(w, v.y, acc.y);
  acc.z = fmaf(w, v.z, acc.z);
  acc.w = fmaf(w, v.w, acc.w);
}

// Any k: slot by slot.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y, int64_t P, int64_t H,
                                                          const int32_t* __restrict__ pair_index,
                                                          const float* __restrict__ weights, int k,
                                                          uint32_t quads_per_row, uint32_t total,
                                                          float* __restrict__ out, uint16_t* __restrict__ out_bf16) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const uint32_t t = gid / quads_per_row;
  const uint32_t c = gid - t * quads_per_row;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int32_t p = pair_index[(int64_t)t * k + j];
    if (p < 0 || p >= P) continue;  // empty slot (an index past the pairs is treated as one)
    combine_fma(acc, weights[(int64_t)t * k + j], reinterpret_cast<const float4*>(y + (int64_t)p * H)[c]);
  }
  combine_store(acc, t, c, H, out, out_bf16);
}

// k == K, a compile-time constant (and P > 0): all slot indices and weights
// are loaded first, then all K row reads are issued before the first is used,
// so a lane keeps K reads in flight instead of one. Empty slots read row 0 (in
// bounds) and are then left out by a select; the sum is the same slot-order
// chain of FMAs.
template <int K>
__global__ __launch_bounds__(256) void moe_combine_batched_kernel(const float* __restrict__ y, int64_t P, int64_t H,
                                                                  const int32_t* __restrict__ pair_index,
                                                                  const float* __restrict__ weights,
                                                                  uint32_t quads_per_row, uint32_t total,
                                                                  float* __restrict__ out,
                                                                  uint16_t* __restrict__ out_bf16) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const uint32_t t = gid / quads_per_row;
  const uint32_t c = gid - t * quads_per_row;
  int32_t p[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    p[j] = pair_index[(int64_t)t * K + j];
    w[j] = weights[(int64_t)t * K + j];
  }
  float4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool ok = p[j] >= 0 && p[j] < P;
    v[j] = reinterpret_cast<const float4*>(y + (int64_t)(ok ? p[j] : 0) * H)[c];
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float4 next = acc;
    combine_fma(next, w[j], v[j]);
    if (p[j] >= 0 && p[j] < P) acc = next;
  }
  combine_store(acc, t, c, H, out, out_bf16);
}

}  // namespace

hipError_t launch_moe_combine(const float* y, int64_t P, int64_t H, const int32_t* pair_index, const float* weights,
                              int64_t T, int k, float* out, uint16_t* out_bf16, hipStream_t stream) {
  const uint32_t qpr = (uint32_t)(H / 4);
  const uint32_t total = (uint32_t)(T * qpr);
  const dim3 grid((total + 255) / 256);
  if (P > 0 && k == 8)
    hipLaunchKernelGGL(moe_combine_batched_kernel<8>, grid, dim3(256), 0, stream, y, P, H, pair_index, weights, qpr,
                       total, out, out_bf16);
  else if (P > 0 && k == 4)
    hipLaunchKernelGGL(moe_combine_batched_kernel<4>, grid, dim3(256), 0, stream, y, P, H, pair_index, weights, qpr,
                       total, out, out_bf16);
  else if (P > 0 && k == 2)
    hipLaunchKernelGGL(moe_combine_batched_kernel<2>, grid, dim3(256), 0, stream, y, P, H, pair_index, weights, qpr,
                       total, out, out_bf16);
  else
    hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, stream, y, P, H, pair_index, weights, k, qpr, total,
                       out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gu, int64_t T, int64_t I, uint16_t* h, hipStream_t stream) {
  const uint32_t gpr = (uint32_t)(I / 8);
  const uint32_t total = (uint32_t)(T * gpr);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, gu, I, gpr, total, h);
  return hipGetLastError();
}

}  // namespace sharq
