// Two-path MXFP4 GEMM on gfx950 scaled MFMA.
//
// What it computes (page "SharQ: Bridging Activation Sparsity and FP4
// Quantization for LLM Inference", Abstract and Section 1): a sparse FP4 GEMM
// over the backbone and a dense FP4 GEMM over the residual share one FP4
// weight load, and the residual path accumulates into the sparse output:
//   Y[t][o] = sum_k bb[t][k] W[o][k] + sum_k res[t][k] W[o][k].
//
// gfx950 has no structured-sparse MFMA for FP4 or with MX scales, so the
// backbone runs as a dense scaled MFMA on its dense-masked codes (dropped
// positions hold code 0). Both paths issue V_MFMA_SCALE_F32_32X32X64_F8F6F4
// (FP4 x FP4, one E8M0 scale per lane per 32 K entries) on the SAME weight
// fragment registers into the SAME fp32 accumulator.
//
// Tiling: a 256-thread workgroup computes a 128 (rows) x 256 (outputs) tile;
// wave w covers rows 64*(w&1) .. +64 and outputs 128*(w>>1) .. +128, i.e. 2 x 4
// MFMA tiles of 32 x 32. K advances 128 entries per stage (64 bytes of codes
// per row per operand). Each stage of the backbone tile, residual tile, weight
// tile and their scales is staged in LDS (34 KB, double-buffered); the next
// stage's global loads are in flight while the current stage's 32 MFMAs per
// wave run. LDS rows are 64 bytes; 16-byte chunks are XOR-swizzled by row so
// the 32 lanes that read one MFMA fragment hit distinct banks.
//
// MFMA operand layouts (32x32x64, FP4): lane l holds row (l % 32) and the 32
// consecutive K entries of block (l / 32) of the 64-entry K slice, low nibble
// first, in 4 VGPRs; its scale byte covers exactly those 32 entries. The
// accumulator's register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32.

#include "sharq_device.h"
#include "sharq_internal.h"

namespace sharq {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 64;  // 128 FP4 codes
constexpr int kOffAs = 0;
constexpr int kOffAr = kOffAs + kBM * kRowBytes;
constexpr int kOffW = kOffAr + kBM * kRowBytes;
constexpr int kOffSAs = kOffW + kBN * kRowBytes;
constexpr int kOffSAr = kOffSAs + kBM * 4;
constexpr int kOffSW = kOffSAr + kBM * 4;
constexpr int kStage = kOffSW + kBN * 4;  // 34816 bytes

__device__ __forceinline__ int swz(int row, int part) {
  return row * kRowBytes + ((part ^ ((row >> 1) & 3)) << 4);
}

struct Operands {
  const uint8_t* a_codes[2];   // backbone, residual codes [rows][K/2]
  const uint8_t* a_scales[2];  // [rows][K/32]
  const uint8_t* w_codes;      // [O][K/2]  (already offset to the expert)
  const uint8_t* w_scales;     // [O][K/32]
  int64_t K;
  int64_t O;
  int nsteps;
};

struct Prefetch {
  uint4 a[2][2];  // [path][chunk]
  uint4 w[4];
  uint32_t sa;    // scale dword of one A row of one path
  uint32_t sw;    // scale dword of one W row
};

// 4 scale bytes of one row for K entries [128 s, 128 s + 128); bytes past the
// end of K read as 127 (scale 1.0; their codes are zero).
template <bool kAligned>
__device__ __forceinline__ uint32_t load_scales4(const uint8_t* row, int64_t s, int64_t kblocks) {
  if constexpr (kAligned) {
    return *reinterpret_cast<const uint32_t*>(row + 4 * s);
  } else {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t b = 4 * s + i;
      const uint32_t byte = b < kblocks ? row[b] : 127u;
      v |= byte << (8 * i);
    }
    return v;
  }
}

template <bool kAligned>
__device__ __forceinline__ void load_stage(Prefetch& pf, const Operands& op, int s, int tid,
                                           const int64_t (&a_src)[2], int64_t a_src_scale,
                                           const int64_t (&w_row)[4], int64_t w_row_scale) {
  const int part = tid & 3;
  const int64_t kbytes = op.K >> 1;
  const int64_t col = (int64_t)s * kRowBytes + part * 16;
  const bool col_ok = col < kbytes;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t r = a_src[c];
      pf.a[p][c] = (r >= 0 && col_ok)
                       ? *reinterpret_cast<const uint4*>(op.a_codes[p] + r * kbytes + col)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t r = w_row[c];
    pf.w[c] = (r >= 0 && col_ok) ? *reinterpret_cast<const uint4*>(op.w_codes + r * kbytes + col)
                                 : make_uint4(0, 0, 0, 0);
  }
  const int64_t kblocks = op.K >> 5;
  const int path = tid >> 7;
  pf.sa = a_src_scale >= 0 ? load_scales4<kAligned>(op.a_scales[path] + a_src_scale * kblocks, s, kblocks)
                           : 0x7F7F7F7Fu;
  pf.sw = w_row_scale >= 0 ? load_scales4<kAligned>(op.w_scales + w_row_scale * kblocks, s, kblocks)
                           : 0x7F7F7F7Fu;
}

__device__ __forceinline__ void store_stage(const Prefetch& pf, uint8_t* st, int tid) {
  const int part = tid & 3;
  const int r0 = tid >> 2;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = r0 + 64 * c;
    *reinterpret_cast<uint4*>(st + kOffAs + swz(row, part)) = pf.a[0][c];
    *reinterpret_cast<uint4*>(st + kOffAr + swz(row, part)) = pf.a[1][c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(st + kOffW + swz(r0 + 64 * c, part)) = pf.w[c];
  const int path = tid >> 7;
  *reinterpret_cast<uint32_t*>(st + (path ? kOffSAr : kOffSAs) + 4 * (tid & 127)) = pf.sa;
  *reinterpret_cast<uint32_t*>(st + kOffSW + 4 * tid) = pf.sw;
}

__device__ __forceinline__ v8i frag(const uint8_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

// One 64-entry K slice (SUB selects which half of the 128-entry stage).
template <int SUB>
__device__ __forceinline__ void compute_sub(const uint8_t* st, v16f (&acc)[2][4], int wm, int wn, int lr,
                                            int lh, const uint32_t (&sa)[2][2], const uint32_t (&sw)[4]) {
  v8i fa[2][2], fw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 64 * wm + 32 * i + lr;
    fa[0][i] = frag(st + kOffAs + swz(row, 2 * SUB + lh));
    fa[1][i] = frag(st + kOffAr + swz(row, 2 * SUB + lh));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) fw[j] = frag(st + kOffW + swz(128 * wn + 32 * j + lr, 2 * SUB + lh));
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0][i], fw[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)sa[0][i], 2 * SUB, (int)sw[j]);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[1][i], fw[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)sa[1][i], 2 * SUB, (int)sw[j]);
    }
}

// Shared main loop. `a_src[c]` is the source activation row of the tile row that
// this thread loads for chunk c (-1 past the end), `a_src_scale` the source row
// whose scales it loads, and likewise for the weight rows.
template <bool kAligned>
__device__ __forceinline__ void mainloop(const Operands& op, uint8_t* smem, v16f (&acc)[2][4],
                                         const int64_t (&a_src)[2], int64_t a_src_scale,
                                         const int64_t (&w_row)[4], int64_t w_row_scale) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  Prefetch pf;
  load_stage<kAligned>(pf, op, 0, tid, a_src, a_src_scale, w_row, w_row_scale);
  store_stage(pf, smem, tid);
  __syncthreads();
  for (int s = 0; s < op.nsteps; ++s) {
    const uint8_t* cur = smem + (s & 1) * kStage;
    const bool more = s + 1 < op.nsteps;
    if (more) load_stage<kAligned>(pf, op, s + 1, tid, a_src, a_src_scale, w_row, w_row_scale);
    uint32_t sa[2][2], sw[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 64 * wm + 32 * i + lr;
      sa[0][i] = *reinterpret_cast<const uint32_t*>(cur + kOffSAs + 4 * row) >> (8 * lh);
      sa[1][i] = *reinterpret_cast<const uint32_t*>(cur + kOffSAr + 4 * row) >> (8 * lh);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sw[j] = *reinterpret_cast<const uint32_t*>(cur + kOffSW + 4 * (128 * wn + 32 * j + lr)) >> (8 * lh);
    compute_sub<0>(cur, acc, wm, wn, lr, lh, sa, sw);
    compute_sub<1>(cur, acc, wm, wn, lr, lh, sa, sw);
    if (more) store_stage(pf, smem + ((s + 1) & 1) * kStage, tid);
    __syncthreads();
  }
}

// Plain two-path GEMM: tiles are assigned so that each XCD (workgroups are
// dispatched round-robin over 8 XCDs) receives a contiguous range of tiles;
// inside a range consecutive tiles share a weight column tile.
template <bool kAligned>
__global__ __launch_bounds__(kThreads) void linear_kernel(Operands op, int64_t T, float* __restrict__ y,
                                                          int64_t ldy, int tiles_m, int tiles_total) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  int tile = blockIdx.x;
  if ((tiles_total & 7) == 0) {
    const int per_xcd = tiles_total >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  }
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int tid = threadIdx.x;
  int64_t a_src[2], w_row[4];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t t = m0 + (tid >> 2) + 64 * c;
    a_src[c] = t < T ? t : -1;
  }
  const int64_t ts = m0 + (tid & 127);
  const int64_t a_src_scale = ts < T ? ts : -1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t o = n0 + (tid >> 2) + 64 * c;
    w_row[c] = o < op.O ? o : -1;
  }
  const int64_t os = n0 + tid;
  const int64_t w_row_scale = os < op.O ? os : -1;

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  mainloop<kAligned>(op, smem, acc, a_src, a_src_scale, w_row, w_row_scale);

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t o = n0 + 128 * wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (t < T && o < op.O) y[t * ldy + o] = acc[i][j][r];
      }
    }
}

// Inclusive prefix sum across a 64-lane wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Grouped two-path GEMM over token-sorted expert segments. blockIdx.y is a
// linear index over all (expert, row-tile) pairs; the expert is found by a
// prefix sum of per-expert tile counts. blockIdx.x is the output column tile.
template <bool kAligned>
__global__ __launch_bounds__(kThreads) void linear_grouped_kernel(
    Operands op, const int32_t* __restrict__ a_rows, const int32_t* __restrict__ seg, int E,
    const uint8_t* __restrict__ w_codes_all, const uint8_t* __restrict__ w_scales_all, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  __shared__ int s_info[2];
  const int tid = threadIdx.x;
  const int target = blockIdx.y;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  if (tid < 64) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + tid;
      const int cnt = e < E ? seg[e + 1] - seg[e] : 0;
      const int tiles = (cnt + kBM - 1) / kBM;
      const int incl = wave_inclusive_scan(tiles, tid);
      const int excl = incl - tiles;
      if (e < E && target >= base + excl && target < base + incl) {
        s_info[0] = e;
        s_info[1] = target - base - excl;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;  // uniform across the workgroup
  const int64_t lo = seg[e] + (int64_t)s_info[1] * kBM;
  const int64_t hi = seg[e + 1];
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  op.w_codes = w_codes_all + (int64_t)e * op.O * (op.K >> 1);
  op.w_scales = w_scales_all + (int64_t)e * op.O * (op.K >> 5);

  int64_t a_src[2], w_row[4];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t p = lo + (tid >> 2) + 64 * c;
    a_src[c] = p < hi ? (a_rows ? (int64_t)a_rows[p] : p) : -1;
  }
  const int64_t ps = lo + (tid & 127);
  const int64_t a_src_scale = ps < hi ? (a_rows ? (int64_t)a_rows[ps] : ps) : -1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t o = n0 + (tid >> 2) + 64 * c;
    w_row[c] = o < op.O ? o : -1;
  }
  const int64_t os = n0 + tid;
  const int64_t w_row_scale = os < op.O ? os : -1;

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  mainloop<kAligned>(op, smem, acc, a_src, a_src_scale, w_row, w_row_scale);

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t o = n0 + 128 * wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t p = lo + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (p < hi && o < op.O) y[p * op.O + o] = acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_linear(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  Operands op;
  op.a_codes[0] = bb_codes;
  op.a_codes[1] = res_codes;
  op.a_scales[0] = bb_scales;
  op.a_scales[1] = res_scales;
  op.w_codes = w_codes;
  op.w_scales = w_scales;
  op.K = K;
  op.O = O;
  op.nsteps = (int)((K + 127) / 128);
  const int tiles_m = (int)((T + kBM - 1) / kBM);
  const int tiles_n = (int)((O + kBN - 1) / kBN);
  const int total = tiles_m * tiles_n;
  if (K % 128 == 0)
    hipLaunchKernelGGL(linear_kernel<true>, dim3(total), dim3(kThreads), 0, stream, op, T, y, ldy, tiles_m, total);
  else
    hipLaunchKernelGGL(linear_kernel<false>, dim3(total), dim3(kThreads), 0, stream, op, T, y, ldy, tiles_m, total);
  return hipGetLastError();
}

hipError_t launch_linear_grouped(const uint8_t* bb_codes, const uint8_t* bb_scales,
                                 const uint8_t* res_codes, const uint8_t* res_scales,
                                 const int32_t* a_rows, const int32_t* seg_offsets, int32_t E,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t O,
                                 int64_t K, float* y, hipStream_t stream) {
  Operands op;
  op.a_codes[0] = bb_codes;
  op.a_codes[1] = res_codes;
  op.a_scales[0] = bb_scales;
  op.a_scales[1] = res_scales;
  op.w_codes = w_codes;
  op.w_scales = w_scales;
  op.K = K;
  op.O = O;
  op.nsteps = (int)((K + 127) / 128);
  // every expert contributes ceil(count / 128) row tiles: at most P/128 + E in total
  const int64_t tiles_m_bound = (P + kBM - 1) / kBM + E;
  const int tiles_n = (int)((O + kBN - 1) / kBN);
  const dim3 grid(tiles_n, (unsigned)tiles_m_bound);
  if (K % 128 == 0)
    hipLaunchKernelGGL(linear_grouped_kernel<true>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets, E,
                       w_codes, w_scales, y);
  else
    hipLaunchKernelGGL(linear_grouped_kernel<false>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets,
                       E, w_codes, w_scales, y);
  return hipGetLastError();
}

}  // namespace sharq
