// SharQ on NVFP4 for gfx950: the prepare operator, the weight quantiser and
// the two-path GEMM with NVFP4 operands.
//
// What it computes (page "SharQ: Bridging Activation Sparsity and FP4
// Quantization for LLM Inference", Abstract: the method generalises to NVFP4
// as well as MXFP4): the same decomposition as the MXFP4 kernels (N:M mask,
// backbone, residual against the quantised backbone, both paths against one
// FP4 weight), with NVFP4 codes. The pages name NVFP4 without defining it; its
// public definition is used: E2M1 codes in 16-entry blocks along K, one FP8
// E4M3 scale per block, one fp32 scale per tensor (the activation's shared by
// backbone and residual, the weight's its own).
//
// Coding of a 16-entry block (all fp32, round to nearest even):
//   v = amax / fp32(6 s_t); scale = the E4M3 value nearest to v (ties to the
//   even code, 448 for anything larger); d = fp32(e4m3(scale) s_t);
//   code = the E2M1 code nearest to fp32(x / d), saturated at 6, sign kept on
//   zero (every entry a signed zero when d == 0).
// Residual: r = fp32(x' - fp32(e2m1 * e4m3 * s_a)).
//
// Layout (stage-major, as the MXFP4 tensors): codes [G][rows][64], K entry k
// of stage g at byte k / 2 of the row's 64 bytes (even k in the low nibble);
// scales [G][rows][8], the E4M3 byte of the stage's 16-block j at byte j.
// G = ceil(K / 128); bytes past K are zero.
//
// The GEMM: gfx950's scaled FP4 MFMA takes only power-of-two (E8M0) scales per
// 32 entries, while an NVFP4 entry times its E4M3 scale has up to 6
// significant bits. So the codes are widened to fp16, where every such product
// is exact: the converter V_CVT_SCALEF32_PK_F16_FP4 gives the E2M1 values,
// V_CVT_SCALEF32_PK_F16_FP8 the block scales times 2^-4 (keeping every product
// a normal fp16 number), and one packed fp16 multiply forms code x scale.
// V_MFMA_F32_32X32X16_F16 then accumulates both paths in fp32; the epilogue
// multiplies by 2^8 s_a s_w.

#include "prepare_block.h"
#include "prepare_io.h"
#include "sharq_internal.h"

namespace sharq {
namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Block coding
// ---------------------------------------------------------------------------

// E4M3 byte of the value nearest to v >= 0, ties to the even code; 0x7E (448)
// for v >= 448 and +inf. Normal E4M3 values below 448 have exponents -6..8 and
// a step of 2^(e-3); below 2^-6 the step is 2^-9. Scaling by a power of two is
// exact and rint rounds half to even, so each branch is one exact rounding.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  const int f = (int)(__float_as_uint(v) >> 23);  // biased exponent (v >= 0)
  if (f < 127 - 6) return (uint32_t)__builtin_rintf(v * 512.0f);  // 0..8; 8 is byte 0x08, 2^-6
  const int e = f - 127;                                           // -6..8
  const uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(v, 3 - e));  // 8..16; 16 carries into e + 1
  return (uint32_t)((e + 7) << 3) + q - 8u;
}

// Value of an E4M3 byte (sign clear, not 0x7F): 2^(e-7) (1 + m/8), or m 2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// fp32(x / d), the correctly rounded quotient, from rd = fp64(1 / d): the
// exact quotient of two fp32 numbers is either an fp32 rounding midpoint's
// neighbour at a relative distance of at least 2^-49 or not near one at all
// (x - M d is a non-zero multiple of M d's last bit, and it cannot be zero
// since M's odd 25-bit significand cannot divide x's 24-bit one), while
// fp64(x * rd) is within a relative 2^-52 + 2^-106 of it; rounding that to
// fp32 therefore gives the same result. Quotients in the fp32 subnormal range
// are far below E2M1's first midpoint (0.25), so they code as a signed zero
// either way. One fp64 multiply per entry instead of a division sequence.
__device__ __forceinline__ float nv_quotient(float x, double rd) { return (float)((double)x * rd); }

// E2M1 codes of 16 entries (8 bytes, low nibble first) for divisor d.
__device__ __forceinline__ uint2 nv_codes16(const float* v, float d) {
  // d == 0: a reciprocal of 0 makes every quotient x * 0, a signed zero
  const double rd = d > 0.0f ? 1.0 / (double)d : 0.0;
  uint32_t w[2];
#pragma unroll
  for (int dw = 0; dw < 2; ++dw) {
    uint32_t r = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // x / d as fp32, clamped to [-7, 7] (one median; signed zeros pass);
      // the converter saturates everything past 6 to 6, an fp32 overflow
      // of the quotient included
      const float q0 = __builtin_amdgcn_fmed3f(nv_quotient(v[8 * dw + 2 * p], rd), -7.0f, 7.0f);
      const float q1 = __builtin_amdgcn_fmed3f(nv_quotient(v[8 * dw + 2 * p + 1], rd), -7.0f, 7.0f);
      switch (p) {
        case 0: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q0, q1, 1.0f, 0); break;
        case 1: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q0, q1, 1.0f, 1); break;
        case 2: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q0, q1, 1.0f, 2); break;
        default: r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q0, q1, 1.0f, 3); break;
      }
    }
    w[dw] = r;
  }
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ float amax16(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[k]));
  return m;
}

struct Nv16 {
  uint2 codes;
  uint32_t scale;
  float sdec;  // e4m3 value of the scale
};

__device__ __forceinline__ Nv16 nv_block16(const float* v, float s_t, float t6) {
  Nv16 b;
  b.scale = e4m3_rne_sat(amax16(v) / t6);
  b.sdec = e4m3_value(b.scale);
  b.codes = nv_codes16(v, b.sdec * s_t);
  return b;
}

// r = fp32(x - fp32(e2m1 * e4m3 * s_t)) for the 16 entries of a coded block.
__device__ __forceinline__ void nv_residual16(const float* x, const Nv16& b, float s_t, float* r) {
#pragma clang fp contract(off)
  const uint32_t w[2] = {b.codes.x, b.codes.y};
#pragma unroll
  for (int dw = 0; dw < 2; ++dw) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      v2f e;
      switch (p) {
        case 0: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[dw], 1.0f, 0); break;
        case 1: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[dw], 1.0f, 1); break;
        case 2: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[dw], 1.0f, 2); break;
        default: e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[dw], 1.0f, 3); break;
      }
      const int k = 8 * dw + 2 * p;
      const float q0 = (e[0] * b.sdec) * s_t;  // e2m1 * e4m3 is exact; one rounding for * s_t
      const float q1 = (e[1] * b.sdec) * s_t;
      r[k] = x[k] - q0;
      r[k + 1] = x[k + 1] - q1;
    }
  }
}

__device__ __forceinline__ int64_t nv_scale_offset(int64_t row, uint32_t chunk, int64_t rows) {
  return (int64_t)(chunk >> 2) * rows * 8 + row * 8 + (chunk & 3) * 2;
}

// ---------------------------------------------------------------------------
// Prepare and weight quantiser: one lane per 32-entry chunk (two NVFP4 blocks),
// lanes mapped as in the MXFP4 prepare (block_of_lane).
// ---------------------------------------------------------------------------

template <int N, int M, bool kGamma>
__global__ __launch_bounds__(256) void prepare_nvfp4_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, uint32_t chunks_per_row,
    uint32_t stages, uint32_t rows, float s_t, uint8_t* __restrict__ bb_codes, uint8_t* __restrict__ bb_scales,
    uint8_t* __restrict__ res_codes, uint8_t* __restrict__ res_scales, uint8_t* __restrict__ mask_out) {
  const BlockOfLane lb = block_of_lane(stages, chunks_per_row, rows);
  if (!lb.row_ok) return;
  if (!lb.block_ok) {  // padding of the last stage: zero codes and scales
    *reinterpret_cast<uint4*>(bb_codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(res_codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint16_t*>(bb_scales + nv_scale_offset(lb.t, lb.b, rows)) = 0;
    *reinterpret_cast<uint16_t*>(res_scales + nv_scale_offset(lb.t, lb.b, rows)) = 0;
    return;
  }
  uint4 raw[4];
  load_block(x + (int64_t)lb.t * ldx + (int64_t)lb.b * 32, raw);
  float xv[32];
  widen_block(raw, xv);
  if constexpr (kGamma) {
    uint4 graw[4];
    load_block(gamma + (int64_t)lb.b * 32, graw);
    times_gamma(xv, graw);
  }
  float xs[32];
  const uint32_t keep = select_block<N, M, kGamma>(xv, xs);
  const float t6 = 6.0f * s_t;
  Nv16 bb[2], rs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bb[h] = nv_block16(xs + 16 * h, s_t, t6);
    float r[16];
    nv_residual16(xv + 16 * h, bb[h], s_t, r);
    rs[h] = nv_block16(r, s_t, t6);
  }
  *reinterpret_cast<uint4*>(bb_codes + code_offset(lb.t, lb.b, rows)) =
      make_uint4(bb[0].codes.x, bb[0].codes.y, bb[1].codes.x, bb[1].codes.y);
  *reinterpret_cast<uint4*>(res_codes + code_offset(lb.t, lb.b, rows)) =
      make_uint4(rs[0].codes.x, rs[0].codes.y, rs[1].codes.x, rs[1].codes.y);
  *reinterpret_cast<uint16_t*>(bb_scales + nv_scale_offset(lb.t, lb.b, rows)) =
      (uint16_t)(bb[0].scale | (bb[1].scale << 8));
  *reinterpret_cast<uint16_t*>(res_scales + nv_scale_offset(lb.t, lb.b, rows)) =
      (uint16_t)(rs[0].scale | (rs[1].scale << 8));
  if (mask_out) reinterpret_cast<uint32_t*>(mask_out)[(int64_t)lb.t * chunks_per_row + lb.b] = keep;
}

__global__ __launch_bounds__(256) void quantize_nvfp4_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                             uint32_t chunks_per_row, uint32_t stages, uint32_t rows,
                                                             float s_t, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const BlockOfLane lb = block_of_lane(stages, chunks_per_row, rows);
  if (!lb.row_ok) return;
  if (!lb.block_ok) {
    *reinterpret_cast<uint4*>(codes + code_offset(lb.t, lb.b, rows)) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint16_t*>(scales + nv_scale_offset(lb.t, lb.b, rows)) = 0;
    return;
  }
  uint4 raw[4];
  load_block(w + (int64_t)lb.t * ldw + (int64_t)lb.b * 32, raw);
  float v[32];
  widen_block(raw, v);
  const float t6 = 6.0f * s_t;
  const Nv16 b0 = nv_block16(v, s_t, t6), b1 = nv_block16(v + 16, s_t, t6);
  *reinterpret_cast<uint4*>(codes + code_offset(lb.t, lb.b, rows)) =
      make_uint4(b0.codes.x, b0.codes.y, b1.codes.x, b1.codes.y);
  *reinterpret_cast<uint16_t*>(scales + nv_scale_offset(lb.t, lb.b, rows)) = (uint16_t)(b0.scale | (b1.scale << 8));
}

// ---------------------------------------------------------------------------
// Two-path GEMM: 128 x 256 output tiles, 4 waves (2 x 2), each wave 64 x 128
// (2 x 4 MFMA tiles of 32 x 32), one 128-entry K stage per LDS buffer, two
// buffers filled through registers.
// ---------------------------------------------------------------------------

constexpr int kNvBM = 128, kNvBN = 256, kNvThreads = 256;
constexpr int kNvOffAs = 0, kNvOffAr = kNvBM * 64, kNvOffW = 2 * kNvBM * 64;
constexpr int kNvOffSAs = kNvOffW + kNvBN * 64, kNvOffSAr = kNvOffSAs + kNvBM * 8, kNvOffSW = kNvOffSAr + kNvBM * 8;
constexpr int kNvStage = kNvOffSW + kNvBN * 8;  // 36 KB

struct NvOperands {
  const uint8_t *as_c, *as_s, *ar_c, *ar_s, *w_c, *w_s;
  int64_t T, O;
  int stages;
};

// One stage of the tile in registers: 8 x 16 bytes of codes and 2 x 8 bytes of
// scales per thread. Chunk i * 256 + tid of the concatenated code arrays
// [A_s 512 | A_r 512 | W 1024] (16-byte chunks, 4 per row); scale row
// i * 256 + tid of [A_s 128 | A_r 128 | W 256]. Rows past T or O read zeros.
struct NvStageRegs {
  uint4 c[8];
  uint2 s[2];
};

__device__ __forceinline__ void nv_load_stage(const NvOperands& op, int g, int64_t m0, int64_t n0, int tid,
                                              NvStageRegs& r) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = (i & 1) * 256 + tid + (i >= 4 ? ((i - 4) >> 1) * 512 : 0);  // index inside its array
    const int row = idx >> 2, ch = idx & 3;
    const uint8_t* base = i < 2 ? op.as_c : i < 4 ? op.ar_c : op.w_c;
    const int64_t R = i < 4 ? op.T : op.O;
    const int64_t grow = (i < 4 ? m0 : n0) + row;
    r.c[i] = grow < R ? *reinterpret_cast<const uint4*>(base + ((int64_t)g * R + grow) * 64 + ch * 16)
                      : make_uint4(0, 0, 0, 0);
  }
  {
    const bool as = tid < 128;
    const uint8_t* base = as ? op.as_s : op.ar_s;
    const int64_t grow = m0 + (tid & 127);
    r.s[0] = grow < op.T ? *reinterpret_cast<const uint2*>(base + ((int64_t)g * op.T + grow) * 8) : make_uint2(0, 0);
    const int64_t wrow = n0 + tid;
    r.s[1] = wrow < op.O ? *reinterpret_cast<const uint2*>(op.w_s + ((int64_t)g * op.O + wrow) * 8)
                         : make_uint2(0, 0);
  }
}

// LDS code rows are 64 bytes; the 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 2) & 3), so 16 consecutive rows read at one logical chunk cover
// all 64 banks.
__device__ __forceinline__ int nv_chunk(int row, int ch) { return ch ^ ((row >> 2) & 3); }

__device__ __forceinline__ void nv_store_stage(uint8_t* lds, int tid, const NvStageRegs& r) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = (i & 1) * 256 + tid + (i >= 4 ? ((i - 4) >> 1) * 512 : 0);
    const int row = idx >> 2, ch = idx & 3;
    const int off = (i < 2 ? kNvOffAs : i < 4 ? kNvOffAr : kNvOffW) + row * 64 + nv_chunk(row, ch) * 16;
    *reinterpret_cast<uint4*>(lds + off) = r.c[i];
  }
  *reinterpret_cast<uint2*>(lds + (tid < 128 ? kNvOffSAs : kNvOffSAr) + (tid & 127) * 8) = r.s[0];
  *reinterpret_cast<uint2*>(lds + kNvOffSW + tid * 8) = r.s[1];
}

// A lane's block scales of one row for the stage: the 4 blocks covering K
// entries 64 h .. 64 h + 63 (h = lane / 32), as fp16 values times 2^-4.
struct NvScales {
  v2h s01, s23;
};

__device__ __forceinline__ NvScales nv_read_scales(const uint8_t* lds, int scale_off, int row, int h) {
  const uint32_t s = *reinterpret_cast<const uint32_t*>(lds + scale_off + row * 8 + 4 * h);
  return NvScales{__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 0.0625f, false),
                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 0.0625f, true)};
}

// The lane's 16 code bytes of k-step quad Q (k-steps 4 Q .. 4 Q + 3: K entries
// 64 h + 32 Q .. + 31) of one row.
template <int Q>
__device__ __forceinline__ uint4 nv_read_codes(const uint8_t* lds, int code_off, int row, int h) {
  return *reinterpret_cast<const uint4*>(lds + code_off + row * 64 + nv_chunk(row, 2 * h + Q) * 16);
}

// MFMA operand of k-step KS: the lane's 8 entries 64 h + 8 KS .. + 7 (inside
// its block KS / 2), each E2M1 value times the block scale.
template <int KS>
__device__ __forceinline__ v8h nv_frag(uint32_t word, const NvScales& s) {
  const _Float16 sh = (KS >> 1) == 0 ? s.s01[0] : (KS >> 1) == 1 ? s.s01[1] : (KS >> 1) == 2 ? s.s23[0] : s.s23[1];
  const v2h s2 = {sh, sh};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * s2;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t nv_word(const uint4& c, int i) {
  return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w;
}

template <int KS>
__device__ __forceinline__ void nv_kstep(const uint4 (&cs)[2], const uint4 (&cr)[2], const uint4 (&cw)[4],
                                         const NvScales (&ss)[2], const NvScales (&sr)[2], const NvScales (&sw)[4],
                                         v16f (&acc)[2][4]) {
  v8h fw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fw[j] = nv_frag<KS>(nv_word(cw[j], KS & 3), sw[j]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const v8h fs = nv_frag<KS>(nv_word(cs[i], KS & 3), ss[i]);
    const v8h fr = nv_frag<KS>(nv_word(cr[i], KS & 3), sr[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fs, fw[j], acc[i][j], 0, 0, 0);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr, fw[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <int Q>
__device__ __forceinline__ void nv_quad(const uint8_t* lds, const int (&ra)[2], const int (&rw)[4], int h,
                                        const NvScales (&ss)[2], const NvScales (&sr)[2], const NvScales (&sw)[4],
                                        v16f (&acc)[2][4]) {
  uint4 cs[2], cr[2], cw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cs[i] = nv_read_codes<Q>(lds, kNvOffAs, ra[i], h);
    cr[i] = nv_read_codes<Q>(lds, kNvOffAr, ra[i], h);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) cw[j] = nv_read_codes<Q>(lds, kNvOffW, rw[j], h);
  nv_kstep<4 * Q + 0>(cs, cr, cw, ss, sr, sw, acc);
  nv_kstep<4 * Q + 1>(cs, cr, cw, ss, sr, sw, acc);
  nv_kstep<4 * Q + 2>(cs, cr, cw, ss, sr, sw, acc);
  nv_kstep<4 * Q + 3>(cs, cr, cw, ss, sr, sw, acc);
}

__device__ __forceinline__ void nv_compute_stage(const uint8_t* lds, int wm, int wn, int r32, int h,
                                                 v16f (&acc)[2][4]) {
  int ra[2], rw[4];
  NvScales ss[2], sr[2], sw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ra[i] = wm * 64 + i * 32 + r32;
    ss[i] = nv_read_scales(lds, kNvOffSAs, ra[i], h);
    sr[i] = nv_read_scales(lds, kNvOffSAr, ra[i], h);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rw[j] = wn * 128 + j * 32 + r32;
    sw[j] = nv_read_scales(lds, kNvOffSW, rw[j], h);
  }
  nv_quad<0>(lds, ra, rw, h, ss, sr, sw, acc);
  nv_quad<1>(lds, ra, rw, h, ss, sr, sw, acc);
}

// Tile order: each XCD (workgroups are dealt round-robin over 8) gets a
// contiguous range of tiles, walked in groups of 4 row tiles with the row
// tiles innermost, so tiles in flight on one XCD share activation and weight
// tiles in its L2.
__device__ __forceinline__ void nv_tile_of_block(int b, int tiles_m, int tiles_total, int& tm, int& tn) {
  int tile = b;
  if ((tiles_total & 7) == 0) tile = (b & 7) * (tiles_total >> 3) + (b >> 3);
  const int tiles_n = tiles_total / tiles_m;
  const int group = tile / (4 * tiles_n);
  const int first = group * 4;
  const int gsize = min(tiles_m - first, 4);
  const int in_group = tile - group * 4 * tiles_n;
  tm = first + in_group % gsize;
  tn = in_group / gsize;
}

__global__ __launch_bounds__(kNvThreads) void linear_nvfp4_kernel(NvOperands op, float out_scale,
                                                                    float* __restrict__ y, int64_t ldy, int tiles_m,
                                                                    int tiles_total) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kNvStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, r32 = lane & 31, h = lane >> 5;
  int tm, tn;
  nv_tile_of_block(blockIdx.x, tiles_m, tiles_total, tm, tn);
  const int64_t m0 = (int64_t)tm * kNvBM, n0 = (int64_t)tn * kNvBN;

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  NvStageRegs regs;
  nv_load_stage(op, 0, m0, n0, tid, regs);
  nv_store_stage(lds, tid, regs);
  __syncthreads();
  for (int g = 0; g < op.stages; ++g) {
    const bool more = g + 1 < op.stages;
    if (more) nv_load_stage(op, g + 1, m0, n0, tid, regs);
    nv_compute_stage(lds + (g & 1) * kNvStage, wm, wn, r32, h, acc);
    // buffer (g + 1) & 1 was last read in stage g - 1, before the barrier
    if (more) nv_store_stage(lds + ((g + 1) & 1) * kNvStage, tid, regs);
    __syncthreads();
  }

  // C layout of a 32 x 32 tile: lane l holds column l % 32 and rows
  // 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + r32;
      if (col >= op.O) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        if (row < op.T) y[row * ldy + col] = acc[i][j][e] * out_scale;
      }
    }
}

}  // namespace

hipError_t launch_prepare_nvfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma, int n,
                                int m, float s_t, uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes,
                                uint8_t* res_scales, uint8_t* mask, hipStream_t stream) {
  const uint32_t chunks = (uint32_t)(K / 32), stages = (uint32_t)((K + 127) / 128);
  const uint32_t bands = (uint32_t)((T + 15) / 16);
  const uint32_t waves = bands * stages;
  const dim3 grid((waves + 3) / 4), block(256);
#define SHARQ_NV_PREP(NN, MM, G)                                                                                  \
  hipLaunchKernelGGL((prepare_nvfp4_kernel<NN, MM, G>), grid, block, 0, stream, x, ldx, gamma, chunks, stages,   \
                     (uint32_t)T, s_t, bb_codes, bb_scales, res_codes, res_scales, mask)
  if (n == 2 && m == 4) {
    if (gamma) SHARQ_NV_PREP(2, 4, true); else SHARQ_NV_PREP(2, 4, false);
  } else {
    if (gamma) SHARQ_NV_PREP(8, 16, true); else SHARQ_NV_PREP(8, 16, false);
  }
#undef SHARQ_NV_PREP
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const uint16_t* w, int64_t O, int64_t K, int64_t ldw, float s_t, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
  const uint32_t chunks = (uint32_t)(K / 32), stages = (uint32_t)((K + 127) / 128);
  const uint32_t waves = (uint32_t)((O + 15) / 16) * stages;
  hipLaunchKernelGGL(quantize_nvfp4_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, w, ldw, chunks, stages,
                     (uint32_t)O, s_t, codes, scales);
  return hipGetLastError();
}

hipError_t launch_linear_nvfp4(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                               const uint8_t* res_scales, float s_a, const uint8_t* w_codes, const uint8_t* w_scales,
                               float s_w, int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                               hipStream_t stream) {
  NvOperands op;
  op.as_c = bb_codes; op.as_s = bb_scales; op.ar_c = res_codes; op.ar_s = res_scales;
  op.w_c = w_codes; op.w_s = w_scales;
  op.T = T; op.O = O;
  op.stages = (int)((K + 127) / 128);
  const int tiles_m = (int)((T + kNvBM - 1) / kNvBM), tiles_n = (int)((O + kNvBN - 1) / kNvBN);
  const int total = tiles_m * tiles_n;
  // each fp16 operand carries a factor 2^-4
  const float out_scale = (s_a * s_w) * 256.0f;
  hipLaunchKernelGGL(linear_nvfp4_kernel, dim3(total), dim3(kNvThreads), 0, stream, op, out_scale, y, ldy, tiles_m,
                     total);
  return hipGetLastError();
}

}  // namespace sharq
