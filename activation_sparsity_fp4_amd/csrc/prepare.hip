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
#include "prepare_io.h"
#include "sharq_internal.h"

namespace sharq {

// Selection, quantisation and the stores of one block of x'. kLowBits: x'
// may carry more than bf16's 8 significant bits (a product with gamma).
template <int N, int M, bool kLowBits>
__device__ __forceinline__ void prepare_store(const float (&xv)[32], uint32_t t, uint32_t b,
                                              uint32_t blocks_per_row, uint32_t rows,
                                              uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
                                              uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales,
                                              uint8_t* __restrict__ mask_out) {
  const PreparedBlock pb = prepare_block<N, M, kLowBits>(xv);
  *reinterpret_cast<uint4*>(bb_codes + code_offset(t, b, rows)) = pb.c_bb;
  *reinterpret_cast<uint4*>(res_codes + code_offset(t, b, rows)) = pb.c_rs;
  bb_scales[scale_index(t, b, rows)] = (uint8_t)pb.e_bb;
  res_scales[scale_index(t, b, rows)] = (uint8_t)pb.e_rs;
  if (mask_out) reinterpret_cast<uint32_t*>(mask_out)[(int64_t)t * blocks_per_row + b] = pb.keep;
}

__device__ __forceinline__ void zero_block(uint32_t t, uint32_t b, uint32_t rows, uint8_t* __restrict__ bb_codes,
                                           uint8_t* __restrict__ bb_scales, uint8_t* __restrict__ res_codes,
                                           uint8_t* __restrict__ res_scales) {
  *reinterpret_cast<uint4*>(bb_codes + code_offset(t, b, rows)) = make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(res_codes + code_offset(t, b, rows)) = make_uint4(0, 0, 0, 0);
  bb_scales[scale_index(t, b, rows)] = 0;
  res_scales[scale_index(t, b, rows)] = 0;
}

// The whole operator without the norm: x' = x (times gamma when given).
// A work item is one wave's share of block_of_item: a 16-row band times one
// 128-entry stage. The grid holds about as many waves as the chip keeps
// resident, and wave w walks items w, w + W, w + 2W, ... (W waves in all),
// issuing the loads of its next item before coding the current one, so the
// HBM reads of one item overlap the VALU work of the one before (a wave per
// item would read, compute and store in lock step with every other wave).
template <int N, int M, bool kGamma>
__global__ __launch_bounds__(256) void prepare_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma,
    uint32_t blocks_per_row, uint32_t stages, uint32_t rows, uint32_t items,
    uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
    uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales,
    uint8_t* __restrict__ mask_out) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t nwaves = (gridDim.x * blockDim.x) >> 6;
  uint32_t item = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);  // wave-uniform
  if (item >= items) return;  // whole waves
  // Loads are unconditional (a lane without a block reads block 0 of row 0,
  // the last item reads itself again) so that no branch hides from the
  // compiler how many loads are in flight: it then waits for exactly the
  // current item's loads, never for the next item's.
  auto load = [&](const BlockOfLane& lb, uint4 (&raw)[4], uint4 (&graw)[4]) {
    const int64_t t = lb.block_ok ? lb.t : 0, b = lb.block_ok ? lb.b : 0;
    load_block(x + t * ldx + b * kBlock, raw);
    if constexpr (kGamma) load_block(gamma + b * kBlock, graw);
  };
  // One step: issue the next item's loads into (nraw, ngraw), code the
  // current item from (raw, graw). Returns false after the last item. The
  // loop below alternates the two register sets, so no copy of an in-flight
  // load's destination forces a wait.
  auto step = [&](BlockOfLane& lb, const uint4 (&raw)[4], const uint4 (&graw)[4], uint4 (&nraw)[4],
                  uint4 (&ngraw)[4]) {
    const uint32_t next = item + nwaves;
    const bool more = next < items;  // wave-uniform
    const BlockOfLane nb = block_of_item(more ? next : item, lane, stages, blocks_per_row, rows);
    load(nb, nraw, ngraw);
    if (lb.block_ok) {
      float xv[32];
      widen_block(raw, xv);
      if constexpr (kGamma) times_gamma(xv, graw);
      prepare_store<N, M, kGamma>(xv, lb.t, lb.b, blocks_per_row, rows, bb_codes, bb_scales, res_codes,
                                  res_scales, mask_out);
    } else if (lb.row_ok) {
      zero_block(lb.t, lb.b, rows, bb_codes, bb_scales, res_codes, res_scales);  // partial last stage
    }
    item = next;
    lb = nb;
    return more;
  };
  BlockOfLane lb = block_of_item(item, lane, stages, blocks_per_row, rows);
  uint4 raw0[4], graw0[4], raw1[4], graw1[4];
  load(lb, raw0, graw0);
  while (step(lb, raw0, graw0, raw1, graw1) && step(lb, raw1, graw1, raw0, graw0)) {
  }
}

// x_n = bf16(x * r) for the 32 entries of a block (round to nearest even,
// two entries per hardware conversion).
__device__ __forceinline__ void normalize_block(float (&xv)[32], float r) {
#pragma unroll
  for (int k = 0; k < 32; k += 2) {
    const uint32_t w = bf16x2_rne(xv[k] * r, xv[k + 1] * r);
    xv[k] = bf16_lo(w);
    xv[k + 1] = bf16_hi(w);
  }
}

// Sum of the 32 squares of a block in float64, one after the other in index
// order (each square of a bf16 value is exact in float64, so the fused
// multiply-add rounds as the plain sum does).
__device__ __forceinline__ double block_sum_sq(const uint4 (&raw)[4]) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
      s = s + lo * lo;
      s = s + hi * hi;
    }
  }
  return s;
}

// Full RMSNorm absorption for rows of at most 64 Q blocks (K <= 2048 Q),
// one wave per row and no LDS or barrier. Lane l owns blocks l + 64 q
// (q < Q), so each chunk of 64 consecutive blocks is one 64-lane shuffle-down
// tree, which is the pairwise tree over those blocks in index order; the
// chunk roots then combine pairwise (Q is 1 or 2), and blocks past the row
// add exact zeros. The sum, r and the coded blocks are those of
// prepare_rms_kernel bit for bit. Waves walk rows w, w + W, ... and load the
// next row before coding the current one, so one row's HBM reads overlap the
// previous row's arithmetic (measured 3% faster than prepare_rms_kernel on
// the 2048 x 4096 input: 9.8 against 10.15 us).
template <int N, int M, bool kGamma, int Q>
__global__ __launch_bounds__(256) void prepare_rms_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, uint32_t K, uint32_t rows,
    float eps, float* __restrict__ r_out, uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
    uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales, uint8_t* __restrict__ mask_out) {
  static_assert(Q == 1 || Q == 2, "one or two 64-block chunks per row");
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t nwaves = (gridDim.x * blockDim.x) >> 6;
  uint32_t t = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);  // wave-uniform row
  if (t >= rows) return;  // whole waves
  const uint32_t nb = K / kBlock, nblk_padded = (nb + 3) & ~3u;
  // Loads are unconditional (a lane past the row reads block 0 of it again,
  // the last row is read again after itself), so that the compiler waits for
  // exactly the current row's loads and never for the next row's.
  auto load = [&](uint32_t row, uint4 (&raw)[Q][4]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint32_t b = lane + 64 * q;
      load_block(x + (int64_t)row * ldx + (int64_t)(b < nb ? b : 0) * kBlock, raw[q]);
    }
  };
  auto step = [&](const uint4 (&raw)[Q][4], uint4 (&nraw)[Q][4]) {
    const uint32_t next = t + nwaves;
    const bool more = next < rows;  // wave-uniform
    load(more ? next : t, nraw);
    double root = 0.0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      double s = lane + 64 * q < nb ? block_sum_sq(raw[q]) : 0.0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) s = s + __shfl_down(s, d, 64);
      const double chunk = __shfl(s, 0, 64);
      root = q == 0 ? chunk : root + chunk;
    }
    const float r = (float)(1.0 / sqrt(root / (double)K + (double)eps));
    if (lane == 0) r_out[t] = r;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint32_t b = lane + 64 * q;
      if (b < nb) {
        float xv[32];
        widen_block(raw[q], xv);
        normalize_block(xv, r);
        if constexpr (kGamma) {  // gamma is re-read per block (cached): holding it costs occupancy
          uint4 graw[4];
          load_block(gamma + (int64_t)b * kBlock, graw);
          times_gamma(xv, graw);
        }
        prepare_store<N, M, kGamma>(xv, t, b, nb, rows, bb_codes, bb_scales, res_codes, res_scales, mask_out);
      } else if (b < nblk_padded) {
        zero_block(t, b, rows, bb_codes, bb_scales, res_codes, res_scales);  // partial last stage
      }
    }
    t = next;
    return more;
  };
  uint4 raw0[Q][4], raw1[Q][4];
  load(t, raw0);
  while (step(raw0, raw1) && step(raw1, raw0)) {
  }
}

// Full RMSNorm absorption (page "SharQ: ...", Abstract: the fused prepare
// absorbs the layer norm): per row r = 1 / sqrt(S / K + eps), then
// x' = bf16(x * r) (times gamma when given) goes through the same per-block
// prepare.
//
// S, the row's sum of squares, is accumulated in float64 in a fixed order so
// that r is reproducible bit for bit: the 32 squares of each MX block one
// after the other in index order (each square of a bf16 value is exact in
// float64), then the block sums by a pairwise tree over blocks in index order
// (adjacent pairs, level by level, padded with zero blocks to a power of two).
// Mean, eps, sqrt and the reciprocal are correctly rounded float64
// operations; r is rounded to float32.
//
// One workgroup (4 waves) owns 4 rows and walks all of K, so x is read from
// HBM once. A wave step covers a chunk of 16 consecutive blocks of each of
// the 4 rows (lane l: row l / 16, block 16 * chunk + l % 16); chunks go to the
// waves round-robin. Pass 1 sums each block and folds the 16 block sums of a
// row by a shuffle-down tree inside the lane's 16-lane segment, which is the
// pairwise tree over that aligned chunk. Pass 2 (wave w, row w) folds the
// chunk sums the same way over 64 lanes per round and combines rounds with a
// binary-counter stack, which completes the tree. Leaves past the last block
// add exact zeros (the sums are non-negative), so padding further than the
// next power of two changes nothing. Pass 3 prepares the blocks; the first
// kHold chunks of each wave stay in registers from pass 1, later ones are
// read again (the workgroup's own rows, still in L2).
constexpr int kRmsRows = 4;
constexpr uint32_t kRmsMaxChunks = 256;  // K <= 131072
constexpr int kRmsHold = 2;

template <int N, int M, bool kGamma>
__global__ __launch_bounds__(256) void prepare_rms_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, uint32_t K, uint32_t rows,
    float eps, float* __restrict__ r_out, uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
    uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales, uint8_t* __restrict__ mask_out) {
  __shared__ double chunk_sum[kRmsRows][kRmsMaxChunks];
  __shared__ float r_row[kRmsRows];
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t t = blockIdx.x * kRmsRows + (lane >> 4);
  const bool row_ok = t < rows;
  const uint32_t nb = K / kBlock, nblk_padded = (nb + 3) & ~3u, nchunks = (nb + 15) / 16;
  const uint16_t* xrow = x + (int64_t)(row_ok ? t : 0) * ldx;

  auto chunk_block = [&](uint32_t c) { return c * 16 + (lane & 15); };
  auto fold_chunk = [&](uint32_t c, const uint4 (&raw)[4]) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
        s = s + lo * lo;  // the product is exact, so a fused multiply-add rounds the same way
        s = s + hi * hi;
      }
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) s = s + __shfl_down(s, d, 16);
    if ((lane & 15) == 0) chunk_sum[lane >> 4][c] = s;
  };
  auto load_chunk = [&](uint32_t c, uint4 (&raw)[4]) {
    const uint32_t b = chunk_block(c);
    if (row_ok && b < nb) {
      load_block(xrow + (int64_t)b * kBlock, raw);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = make_uint4(0, 0, 0, 0);  // squares of zero: exact zeros
    }
  };

  // pass 1: block sums, folded per chunk
  uint4 held[kRmsHold][4];
#pragma unroll
  for (int it = 0; it < kRmsHold; ++it) {
    const uint32_t c = wave + 4 * it;
    if (c < nchunks) {
      load_chunk(c, held[it]);
      fold_chunk(c, held[it]);
    }
  }
  for (uint32_t c = wave + 4 * kRmsHold; c < nchunks; c += 4) {
    uint4 raw[4];
    load_chunk(c, raw);
    fold_chunk(c, raw);
  }
  __syncthreads();

  // pass 2: wave w completes the tree of row w
  {
    const uint32_t rounds = (nchunks + 63) / 64;
    uint32_t npad = 1;
    while (npad < rounds) npad <<= 1;
    double stack[3];
    double root = 0.0;
    for (uint32_t rd = 0; rd < npad; ++rd) {
      const uint32_t c = rd * 64 + lane;
      double s = c < nchunks ? chunk_sum[wave][c] : 0.0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) s = s + __shfl_down(s, d, 64);
      double cur = __shfl(s, 0, 64);
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        if ((rd >> l) & 1u) {
          cur = stack[l] + cur;
        } else {
          stack[l] = cur;
          break;
        }
      }
      root = cur;
    }
    if (lane == 0) {
      const float r = (float)(1.0 / sqrt(root / (double)K + (double)eps));
      r_row[wave] = r;
      const uint32_t tw = blockIdx.x * kRmsRows + wave;
      if (tw < rows) r_out[tw] = r;
    }
  }
  __syncthreads();

  // pass 3: prepare bf16(x * r)
  const float r = r_row[lane >> 4];
  auto emit = [&](uint32_t c, const uint4 (&raw)[4]) {
    const uint32_t b = chunk_block(c);
    if (!row_ok || b >= nblk_padded) return;
    if (b >= nb) {
      zero_block(t, b, rows, bb_codes, bb_scales, res_codes, res_scales);  // partial last stage
      return;
    }
    float xv[32];
    widen_block(raw, xv);
    normalize_block(xv, r);
    if constexpr (kGamma) {
      uint4 graw[4];
      load_block(gamma + (int64_t)b * kBlock, graw);
      times_gamma(xv, graw);
    }
    prepare_store<N, M, kGamma>(xv, t, b, nb, rows, bb_codes, bb_scales, res_codes, res_scales, mask_out);
  };
#pragma unroll
  for (int it = 0; it < kRmsHold; ++it) {
    const uint32_t c = wave + 4 * it;
    if (c < nchunks) emit(c, held[it]);
  }
  for (uint32_t c = wave + 4 * kRmsHold; c < nchunks; c += 4) {
    uint4 raw[4];
    load_chunk(c, raw);
    emit(c, raw);
  }
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

// Compute units of the current device (queried once per device).
static int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Waves of a 256-thread kernel the current device keeps resident at once
// (occupancy per CU times CUs), cached per device in `cache`.
static uint64_t resident_waves(const void* kernel, int (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0) != hipSuccess || blocks <= 0)
      blocks = 2;
    cache[dev] = blocks;
  }
  return (uint64_t)cache[dev] * 4 * (uint64_t)cu_count();
}

hipError_t launch_prepare(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma,
                          float rms_eps, float* rms_scale, int n, int m, uint8_t* bb_codes, uint8_t* bb_scales,
                          uint8_t* res_codes, uint8_t* res_scales, uint8_t* mask, hipStream_t stream) {
  if (rms_scale && K <= 4096) {
    // one wave per row; at most as many waves as the chip keeps resident (each
    // then walks several rows), whole 4-wave workgroups
#define SHARQ_PREP_ROWS(NN, MM, GG, QQ)                                                                             \
  do {                                                                                                             \
    static int resident[64] = {};                                                                                  \
    const uint64_t cap = resident_waves(reinterpret_cast<const void*>(&prepare_rms_rows_kernel<NN, MM, GG, QQ>),   \
                                        resident);                                                                 \
    const uint64_t per_wave = ((uint64_t)T + cap - 1) / cap;                                                       \
    const uint64_t waves = ((uint64_t)T + per_wave - 1) / per_wave;                                                \
    hipLaunchKernelGGL((prepare_rms_rows_kernel<NN, MM, GG, QQ>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, \
                       stream, x, ldx, gamma, (uint32_t)K, (uint32_t)T, rms_eps, rms_scale, bb_codes, bb_scales,   \
                       res_codes, res_scales, mask);                                                               \
  } while (0)
#define SHARQ_PREP_ROWS_Q(NN, MM, GG) \
  if (K <= 2048) SHARQ_PREP_ROWS(NN, MM, GG, 1); else SHARQ_PREP_ROWS(NN, MM, GG, 2)
    if (n == 2 && m == 4) {
      if (gamma) SHARQ_PREP_ROWS_Q(2, 4, true); else SHARQ_PREP_ROWS_Q(2, 4, false);
    } else {
      if (gamma) SHARQ_PREP_ROWS_Q(8, 16, true); else SHARQ_PREP_ROWS_Q(8, 16, false);
    }
#undef SHARQ_PREP_ROWS_Q
#undef SHARQ_PREP_ROWS
    return hipGetLastError();
  }
  if (rms_scale) {
    const dim3 grid((unsigned)((T + kRmsRows - 1) / kRmsRows)), block(256);
#define SHARQ_PREP_RMS(NN, MM, GG)                                                                          \
  hipLaunchKernelGGL((prepare_rms_kernel<NN, MM, GG>), grid, block, 0, stream, x, ldx, gamma, (uint32_t)K, \
                     (uint32_t)T, rms_eps, rms_scale, bb_codes, bb_scales, res_codes, res_scales, mask)
    if (n == 2 && m == 4) {
      if (gamma) SHARQ_PREP_RMS(2, 4, true); else SHARQ_PREP_RMS(2, 4, false);
    } else {
      if (gamma) SHARQ_PREP_RMS(8, 16, true); else SHARQ_PREP_RMS(8, 16, false);
    }
#undef SHARQ_PREP_RMS
    return hipGetLastError();
  }
  const uint32_t bpr = (uint32_t)(K / kBlock);
  const uint32_t stages = (uint32_t)((K + 127) / 128);
  const uint64_t items = lanes_for(T, K) / 64;
  // Waves in the grid: at most what the chip keeps resident at this
  // variant's register use, each walking the same number of items; small
  // grids take one wave per workgroup so that more CUs take part.
#define SHARQ_PREP(NN, MM, GG)                                                                                    \
  do {                                                                                                            \
    static int resident[64] = {};                                                                                 \
    const uint64_t cap = resident_waves(reinterpret_cast<const void*>(&prepare_kernel<NN, MM, GG>), resident);    \
    const uint64_t per_wave = (items + cap - 1) / cap;                                                            \
    const uint64_t waves = (items + per_wave - 1) / per_wave;                                                     \
    const unsigned threads = waves >= 4 * (uint64_t)cu_count() ? 256 : 64;                                        \
    hipLaunchKernelGGL((prepare_kernel<NN, MM, GG>), dim3((unsigned)((waves * 64 + threads - 1) / threads)),      \
                       dim3(threads), 0, stream, x, ldx, gamma, bpr, stages, (uint32_t)T, (uint32_t)items, bb_codes, \
                       bb_scales, res_codes, res_scales, mask);                                                   \
  } while (0)
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
