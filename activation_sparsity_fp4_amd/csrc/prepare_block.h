// Per-block arithmetic of the SharQ prepare operator, shared by the prepare
// kernel and the fused gate|up epilogue so that both produce identical bits.
//
// What it computes (page "SharQ: Bridging Activation Sparsity and FP4
// Quantization for LLM Inference", Abstract and Section 1): for one 32-entry
// MX block of x' (the activation after the optional RMSNorm weight), an N:M
// mask keeps the N largest |x'| of every M entries; the kept entries form the
// sparse backbone, coded in MXFP4; the residual x' - dequant(backbone) is
// coded in MXFP4 with its own scale.
//
// Selection: magnitudes are compared as integer bit patterns. When the low
// bits of every |x'| in a block are zero (always for bf16 inputs; for x * gamma
// unless the product is an fp32 subnormal) the group position is folded into
// those low bits, which makes every key unique and orders equal magnitudes by
// lower index. Top-2 of 4 is then a max/min tournament and top-8 of 16 uses two
// 8-key sorting networks and a bitonic half-cleaner. Blocks with non-zero low
// bits take an exact pairwise-rank path instead.
#pragma once

#include "sharq_device.h"
#include "sort_network.h"

namespace sharq {

// Mask bits (one per entry, bit k) of the kept entries of a block for n:m.
template <int N, int M>
__device__ __forceinline__ uint32_t select_fast(const float (&x)[32], float (&xs)[32]) {
  static_assert((N == 2 && M == 4) || (N == 8 && M == 16), "pattern");
  // Entry k is kept when its key is at least the group's N-th largest key;
  // one compare per entry yields both its mask bit and its backbone value
  // (xs[k] = x[k] when kept, 0 otherwise).
  uint32_t mask = 0;
  if constexpr (M == 4) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      uint32_t k[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        k[i] = (__float_as_uint(x[4 * g + i]) & 0x7FFFFFFCu) | (3u - i);
      const uint32_t a = max(k[0], k[1]), b = min(k[0], k[1]);
      const uint32_t c = max(k[2], k[3]), d = min(k[2], k[3]);
      const uint32_t second = max(max(min(a, c), b), d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool kept = k[i] >= second;
        xs[4 * g + i] = kept ? x[4 * g + i] : 0.0f;
        mask |= kept ? 1u << (4 * g + i) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint32_t k[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        k[i] = (__float_as_uint(x[16 * g + i]) & 0x7FFFFFF0u) | (15u - i);
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) { lo[i] = k[i]; hi[i] = k[8 + i]; }
#pragma unroll
      for (int c = 0; c < kSort8Size; ++c) {
        const int i = kSort8[c][0], j = kSort8[c][1];
        const uint32_t p = max(lo[i], lo[j]), q = min(lo[i], lo[j]);
        lo[i] = p; lo[j] = q;
        const uint32_t r = max(hi[i], hi[j]), s = min(hi[i], hi[j]);
        hi[i] = r; hi[j] = s;
      }
      uint32_t thr = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < 8; ++i) thr = min(thr, max(lo[i], hi[7 - i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool kept = k[i] >= thr;
        xs[16 * g + i] = kept ? x[16 * g + i] : 0.0f;
        mask |= kept ? 1u << (16 * g + i) : 0u;
      }
    }
  }
  return mask;
}

// Exact selection for any block: entry i is kept when fewer than N entries of
// its group beat it (larger |x'|, or equal |x'| at a lower index).
template <int N, int M>
__device__ __forceinline__ uint32_t select_exact(const float (&x)[32]) {
  uint32_t mask = 0;
#pragma unroll
  for (int g = 0; g < 32 / M; ++g) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t ai = __float_as_uint(x[M * g + i]) & 0x7FFFFFFFu;
      int beaten = 0;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if (j == i) continue;
        const uint32_t aj = __float_as_uint(x[M * g + j]) & 0x7FFFFFFFu;
        beaten += (aj > ai || (aj == ai && j < i)) ? 1 : 0;
      }
      mask |= (beaten < N ? 1u : 0u) << (M * g + i);
    }
  }
  return mask;
}

// N:M mask bits of one 32-entry block and its backbone xs (kept entries,
// zeros elsewhere). kMaybeLowBits: x' may have non-zero low key bits
// (x * gamma), so the block checks and takes the exact selection when needed.
template <int N, int M, bool kMaybeLowBits>
__device__ __forceinline__ uint32_t select_block(const float (&xv)[32], float (&xs)[32]) {
  if constexpr (kMaybeLowBits) {
    uint32_t low = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) low |= __float_as_uint(xv[k]);
    if (low & (uint32_t)(M - 1)) {
      const uint32_t keep = select_exact<N, M>(xv);
#pragma unroll
      for (int k = 0; k < 32; ++k) xs[k] = (keep >> k) & 1u ? xv[k] : 0.0f;
      return keep;
    }
  }
  return select_fast<N, M>(xv, xs);
}

struct PreparedBlock {
  uint4 c_bb, c_rs;      // backbone and residual E2M1 codes (16 bytes each)
  uint32_t e_bb, e_rs;   // E8M0 scale bytes
  uint32_t keep;         // mask bits, bit k for entry k
};

// One block (kMaybeLowBits as for select_block).
template <int N, int M, bool kMaybeLowBits>
__device__ __forceinline__ PreparedBlock prepare_block(const float (&xv)[32]) {
  PreparedBlock out;
  // N:M selection; xs = the backbone (kept entries, zeros elsewhere)
  float xs[32];
  const uint32_t keep = select_block<N, M, kMaybeLowBits>(xv, xs);

  // backbone: the block's largest |x'| is always kept (each group keeps its
  // maximum), so the backbone scale is the block's plain MX scale
  const uint32_t e_bb = e8m0_from_amax_bits(amax_bits32(xv));
  const float s_bb = scale_from_e8m0(e_bb);
  const uint4 c_bb = quantize32(xs, s_bb);

  // residual against the quantised backbone (exact in fp32)
  float q[32];
  dequantize32(c_bb, s_bb, q);
  float r[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) r[k] = xv[k] - q[k];
  const uint32_t e_rs = e8m0_from_amax_bits(amax_bits32(r));
  const uint4 c_rs = quantize32(r, scale_from_e8m0(e_rs));

  out.c_bb = c_bb;
  out.c_rs = c_rs;
  out.e_bb = e_bb;
  out.e_rs = e_rs;
  out.keep = keep;
  return out;
}

}  // namespace sharq
