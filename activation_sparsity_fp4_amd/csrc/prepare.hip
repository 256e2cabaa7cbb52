// Fused SharQ prepare kernel for gfx950.
//
// What it computes (page "SharQ: Bridging Activation Sparsity and FP4
// Quantization for LLM Inference", Abstract and Section 1): per activation row,
// an online N:M mask keeps the N largest |x'| of every M entries along K
// (x' = x * gamma when the RMSNorm weight is absorbed); the kept entries form a
// sparse backbone coded in MXFP4; the residual x' - dequant(backbone) is coded
// in MXFP4 with its own scales.
//
// Work decomposition: one lane owns one 32-entry MX block of one row, so every
// block reduction (amax, scale) and every N:M group (4 or 16 entries, both
// dividing 32) stays inside the lane's registers and no cross-lane traffic is
// needed. A lane reads 64 contiguous bytes of bf16 (four 16-byte loads) and
// writes 16 + 16 bytes of codes, two scale bytes and a 32-bit mask word (see
// block_of_lane for how lanes map to blocks). The kernel is HBM-bound: 2 bytes read and 1.1875 bytes
// written per element.
//
// Selection and quantisation of a block: prepare_block.h.
//
// Quantisation uses the gfx950 scaled converters (v_cvt_scalef32_pk_fp4_f32,
// v_cvt_scalef32_pk_f32_fp4), whose rounding (nearest-even, saturation at 6,
// sign kept on zero) matches the MXFP4 rule exactly for every finite input.

#include "prepare_block.h"
#include "sharq_internal.h"

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

__device__ __forceinline__ BlockOfLane block_of_lane(uint32_t stages, uint32_t blocks_per_row, uint32_t rows) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t wave = gid >> 6, lane = gid & 63;
  const uint32_t band = wave / stages;
  const uint32_t g = wave - band * stages;
  BlockOfLane r;
  r.t = band * 16 + (lane >> 2);
  r.b = g * 4 + (lane & 3);
  r.row_ok = r.t < rows;
  r.block_ok = r.row_ok && r.b < blocks_per_row;
  return r;
}

template <int N, int M, bool kGamma>
__global__ __launch_bounds__(256) void prepare_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma,
    uint32_t blocks_per_row, uint32_t stages, uint32_t rows,
    uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
    uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales,
    uint8_t* __restrict__ mask_out) {
  const BlockOfLane lb = block_of_lane(stages, blocks_per_row, rows);
  if (!lb.block_ok) {
    // the unused blocks of a last, partial stage are zero
    if (lb.row_ok) {
      *reinterpret_cast<uint4*>(bb_codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(res_codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
      bb_scales[scale_index(lb.t, lb.b, rows)] = 0;
      res_scales[scale_index(lb.t, lb.b, rows)] = 0;
    }
    return;
  }
  const uint32_t t = lb.t, b = lb.b;
  const uint32_t gid = t * blocks_per_row + b;  // row-major block index (mask words)

  // load 32 bf16 (64 B) and widen to fp32
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * ldx + (int64_t)b * kBlock);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src[i];
  float xv[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] = bf16_lo(w[j]);
      xv[8 * i + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  if constexpr (kGamma) {
    const uint4* gsrc = reinterpret_cast<const uint4*>(gamma + (int64_t)b * kBlock);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 gr = gsrc[i];
      const uint32_t w[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] *= bf16_lo(w[j]);
        xv[8 * i + 2 * j + 1] *= bf16_hi(w[j]);
      }
    }
  }

  const PreparedBlock pb = prepare_block<N, M, kGamma>(xv);
  const uint4 c_bb = pb.c_bb, c_rs = pb.c_rs;
  const uint32_t e_bb = pb.e_bb, e_rs = pb.e_rs, keep = pb.keep;

  *reinterpret_cast<uint4*>(bb_codes + code_offset(t, b, rows)) = c_bb;
  *reinterpret_cast<uint4*>(res_codes + code_offset(t, b, rows)) = c_rs;
  bb_scales[scale_index(t, b, rows)] = (uint8_t)e_bb;
  res_scales[scale_index(t, b, rows)] = (uint8_t)e_rs;
  if (mask_out) reinterpret_cast<uint32_t*>(mask_out)[gid] = keep;
}

// Plain MXFP4 coding of bf16 rows (the weight quantiser): same element and
// scale rules, no mask and no residual.
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint32_t blocks_per_row, uint32_t stages, uint32_t rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const BlockOfLane lb = block_of_lane(stages, blocks_per_row, rows);
  if (!lb.block_ok) {
    if (lb.row_ok) {
      *reinterpret_cast<uint4*>(codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
      scales[scale_index(lb.t, lb.b, rows)] = 0;
    }
    return;
  }
  const uint32_t t = lb.t, b = lb.b;
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * ldx + (int64_t)b * kBlock);
  float xv[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 rw = src[i];
    const uint32_t w[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[8 * i + 2 * j] = bf16_lo(w[j]);
      xv[8 * i + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  const uint32_t e = e8m0_from_amax_bits(amax_bits32(xv));
  const uint4 c = quantize32(xv, scale_from_e8m0(e));
  *reinterpret_cast<uint4*>(codes + code_offset(t, b, rows)) = c;
  scales[scale_index(t, b, rows)] = (uint8_t)e;
}

// Threads for the lane map of block_of_lane: one wave per (16-row band, stage).
static inline uint64_t lanes_for(int64_t T, int64_t K) {
  const uint64_t bands = (uint64_t)((T + 15) / 16);
  const uint64_t stages = (uint64_t)((K + 127) / 128);
  return bands * stages * 64;
}

hipError_t launch_prepare(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma,
                          int n, int m, uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes,
                          uint8_t* res_scales, uint8_t* mask, hipStream_t stream) {
  const uint32_t bpr = (uint32_t)(K / kBlock);
  const uint32_t stages = (uint32_t)((K + 127) / 128);
  const uint64_t lanes = lanes_for(T, K);
  // small problems: one wave per workgroup so that more CUs take part
  const unsigned threads = lanes >= (1u << 18) ? 256 : 64;
  const dim3 grid((unsigned)((lanes + threads - 1) / threads)), block(threads);
#define SHARQ_PREP(NN, MM, GG)                                                              \
  hipLaunchKernelGGL((prepare_kernel<NN, MM, GG>), grid, block, 0, stream, x, ldx, gamma,   \
                     bpr, stages, (uint32_t)T, bb_codes, bb_scales, res_codes, res_scales, mask)
  if (n == 2 && m == 4) {
    if (gamma) SHARQ_PREP(2, 4, true); else SHARQ_PREP(2, 4, false);
  } else {
    if (gamma) SHARQ_PREP(8, 16, true); else SHARQ_PREP(8, 16, false);
  }
#undef SHARQ_PREP
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  const uint32_t bpr = (uint32_t)(K / kBlock);
  const uint32_t stages = (uint32_t)((K + 127) / 128);
  const uint64_t lanes = lanes_for(T, K);
  const unsigned threads = lanes >= (1u << 18) ? 256 : 64;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((lanes + threads - 1) / threads)), dim3(threads), 0, stream,
                     x, ldx, bpr, stages, (uint32_t)T, codes, scales);
  return hipGetLastError();
}

}  // namespace sharq
