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
// Tiling: a 256-thread workgroup is 2 x 2 waves; each wave computes WM x WN
// MFMA tiles of 32 x 32, so the workgroup tile is (64 WM) x (64 WN); the
// kernels use 128 x 256 (WM = 2, WN = 4). The activation side carries two
// operands (backbone and residual) against one weight operand, so a tile
// twice as wide as it is tall balances the bytes each stage loads. K advances
// 128 entries per stage (64 bytes of codes per row per operand; with the
// stage-major layout of sharq_device.h one stage of a tile is one contiguous
// run of every operand).
//
// Main path (K % 128 == 0): a ring of 34 KB LDS stages filled by buffer
// loads that write straight into LDS (no register staging); the stages ahead
// of the one being consumed are in flight. Rows past the end of a matrix read
// as zero through the buffer bounds check, and one barrier per stage recycles
// a slot as soon as every wave holds that stage's fragments in registers.
// With a ring of 2 the workgroup needs 68 KB of LDS and at most 128
// accumulator plus 128 other VGPRs per lane, so two workgroups share a CU:
// each SIMD runs two waves of independent tiles, and one tile's barrier
// waits, load issue and output stores overlap the other's MFMAs (measured:
// 15% faster on the Llama-3.1-8B gate|up shape than one workgroup per CU with
// a ring of 4, and 10% faster than 256 x 256 tiles). Problems with fewer
// tiles than CUs take one workgroup per CU and a ring of 4. General path
// (any K % 32 == 0): 2 LDS stages filled through registers.
//
// LDS rows are 64 bytes; the 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 2) & 3), which keeps the rows read by one MFMA fragment on
// distinct banks of the 64-bank LDS.
//
// MFMA operand layouts (32x32x64, FP4): lane l holds row (l % 32) and the 32
// consecutive K entries of block (l / 32) of the 64-entry K slice, low nibble
// first, in 4 VGPRs; its scale byte covers exactly those 32 entries. The
// accumulator's register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32.

#include "prepare_block.h"
#include "sharq_device.h"
#include "sharq_internal.h"
#include "silu.h"

namespace sharq {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 64;            // 128 FP4 codes
constexpr int kLdsBytes = 160 * 1024;    // LDS of one CU
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every bound: reads as 0

// Workgroup tile of NWM x 2 waves (NWM along the rows), each WM x WN MFMA
// tiles of 32 x 32, and the layout of one LDS stage: backbone codes, residual
// codes, weight codes, then the three scale runs (in that order; each
// activation scale run is padded to a multiple of 64 rows, the width of one
// buffer->LDS load).
template <int WM_, int WN_, int RING_, int NWM_ = 2>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, NWM = NWM_;
  static constexpr int kWaves = 2 * NWM, kThreads = 64 * kWaves;
  static constexpr int BM = 32 * WM * NWM, BN = 64 * WN;
  static constexpr int kARunRows = (BM + 63) / 64 * 64;  // rows of one activation scale run
  static constexpr int kOffAs = 0;
  static constexpr int kOffAr = BM * kRowBytes;
  static constexpr int kOffW = 2 * BM * kRowBytes;
  static constexpr int kOffSAs = kOffW + BN * kRowBytes;
  static constexpr int kOffSAr = kOffSAs + kARunRows * 4;
  static constexpr int kOffSW = kOffSAr + kARunRows * 4;
  // buffer->LDS instructions per wave per stage: 1 KB code chunks of each
  // activation operand, of the weight, and 256-byte scale runs (64 rows).
  // When the scale runs do not split evenly over the four waves, the spare
  // instructions read nothing (out of range) into a trash area, so that every
  // wave issues the same number of loads per stage.
  static constexpr int kAChunks = BM / 16 / kWaves;
  static constexpr int kWChunks = BN / 16 / kWaves;
  static constexpr int kSRuns = (2 * kARunRows + BN) / 64;
  static constexpr int kSLoads = (kSRuns + kWaves - 1) / kWaves;
  static constexpr int kLoads = 2 * kAChunks + kWChunks + kSLoads;
  static constexpr int kStage = kOffSW + BN * 4 + 256 * (kWaves * kSLoads - kSRuns);
  static_assert(kAChunks * 16 * kWaves == BM && kWChunks * 16 * kWaves == BN, "whole 1 KB chunks per wave");
  static constexpr int kRing = RING_;
  static constexpr int kOccupancy = kLdsBytes / (kRing * kStage);  // workgroups per CU (LDS bound)
  static_assert(kRing >= 2 && kRing * kStage <= kLdsBytes, "ring");
};
using SmallTile = Tile<2, 4, 2>;  // 128 x 256, 34 KB stages, ring of 2, two workgroups per CU
using DeepTile = Tile<2, 4, 4>;   // 128 x 256, ring of 4, one workgroup per CU
// Decode-sized T: 32 x 256 (T <= 32) and 64 x 256 (T <= 64) tiles of two
// waves, ring of 3, two workgroups per CU. A 128-row tile runs up to 4x the
// MFMA work on zero rows, which at T = 1 took longer than streaming the
// weight (Llama-3.1-70B decode step 0.127 -> 0.097 ms at T = 1).
using DecodeTile = Tile<1, 4, 3, 1>;
using Decode64Tile = Tile<2, 4, 3, 1>;

// LDS chunk swizzle. gfx950 LDS has 64 four-byte banks; a ds_read_b128 of an
// MFMA fragment serves 16 lanes (16 consecutive rows, one 16-byte chunk each)
// per pass, and rows r and r + 4 start on the same bank. XOR-ing the chunk
// index with bits 2..3 of the row spreads those 16 rows over all 64 banks
// (measured: zero SQ_LDS_BANK_CONFLICT cycles).
__device__ __forceinline__ int swz_part(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz(int row, int part) {
  return row * kRowBytes + ((part ^ swz_part(row)) << 4);
}

// An MFMA operand fragment from LDS. The FP4 form of the scaled MFMA reads
// only the low 4 of its 8 operand registers, so the upper half is left
// undefined (no registers are spent on it).
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v8i frag(const uint8_t* p) {
  const v4i v = *reinterpret_cast<const v4i*>(p);
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

struct Operands {
  const uint8_t* a_codes[2];   // backbone, residual codes [G][rows][64] (stage-major)
  const uint8_t* a_scales[2];  // [G][rows][4]
  const uint8_t* w_codes;      // [G][O][64]  (already offset to the expert)
  const uint8_t* w_scales;     // [G][O][4]
  int64_t a_rows_total;        // rows addressable through a_codes (bounds of the buffer view)
  int64_t K;
  int64_t O;
  int nsteps;
};

// Row sources of one output tile: which activation row feeds tile row r, or
// -1 (the row then reads as zeros). A gathered index outside [0, src_rows)
// is -1 as well, so malformed gather contents never address memory outside
// the activation buffers.
struct TileRows {
  int64_t m0;          // first output row of the tile
  int64_t rows_valid;  // output rows of the tile that exist (<= the tile height)
  const int32_t* gather;  // activation row of each output row, or nullptr (identity)
  int64_t src_rows;    // rows of the activation buffers (bound of a gathered index)
  __device__ __forceinline__ int64_t src(int r) const {
    if (r >= rows_valid) return -1;
    const int64_t p = m0 + r;
    if (!gather) return p;
    const int64_t g = gather[p];
    return g >= 0 && g < src_rows ? g : -1;
  }
};

// Weight rows of one output tile: the weight row behind tile column c.
// Plain tiles take rows n0 + c. A fused gate|up tile over h columns
// [h0, h0 + 128) of a weight whose rows are [gate (I rows); up (I rows)]
// alternates 64-row blocks: block b = c / 64 holds the gate (b even) or up
// (b odd) rows of h columns h0 + 64 (b / 2) + c % 64, so each wave's four
// 32-column MFMA tiles are gate, gate, up, up of the same 64 h columns.
struct TileCols {
  int64_t n0;    // first output column (plain) or first h column (gate|up)
  int64_t half;  // 0 for a plain tile, else I
  __device__ __forceinline__ int64_t w_row(int c) const {
    if (half == 0) return n0 + c;
    const int b = c >> 6;
    return ((b & 1) ? half : 0) + n0 + 64 * (b >> 1) + (c & 63);
  }
};

// Fragments and scale dwords of one 64-entry sub-step, held in registers.
template <class C>
struct Frags {
  v8i a[2][C::WM];  // [path][row block]
  v8i w[C::WN];
};
template <class C>
struct Scales {
  uint32_t a[2][C::WM];  // [path][row block]
  uint32_t w[C::WN];
};

template <class C, int SUB>
__device__ __forceinline__ void read_frags(const uint8_t* st, Frags<C>& f, int wm, int wn, int lr, int lh) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
    const int row = 32 * C::WM * wm + 32 * i + lr;
    f.a[0][i] = frag(st + C::kOffAs + swz(row, 2 * SUB + lh));
    f.a[1][i] = frag(st + C::kOffAr + swz(row, 2 * SUB + lh));
  }
#pragma unroll
  for (int j = 0; j < C::WN; ++j)
    f.w[j] = frag(st + C::kOffW + swz(32 * C::WN * wn + 32 * j + lr, 2 * SUB + lh));
}

// The scale dword of a lane's row holds the bytes of the stage's 4 blocks;
// shifted right by 8 * (lane / 32), byte 0 (sub-step 0) and byte 2 (sub-step
// 1) are the blocks of that lane's K half, picked by the MFMA's op_sel.
template <class C>
__device__ __forceinline__ void read_scales(const uint8_t* st, Scales<C>& c, int wm, int wn, int lr, int lh) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
    const int row = 32 * C::WM * wm + 32 * i + lr;
    c.a[0][i] = *reinterpret_cast<const uint32_t*>(st + C::kOffSAs + 4 * row) >> (8 * lh);
    c.a[1][i] = *reinterpret_cast<const uint32_t*>(st + C::kOffSAr + 4 * row) >> (8 * lh);
  }
#pragma unroll
  for (int j = 0; j < C::WN; ++j)
    c.w[j] = *reinterpret_cast<const uint32_t*>(st + C::kOffSW + 4 * (32 * C::WN * wn + 32 * j + lr)) >> (8 * lh);
}

template <class C, int SUB>
__device__ __forceinline__ void mfma_sub(const Frags<C>& f, const Scales<C>& c, v16f (&acc)[C::WM][C::WN]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[0][i], f.w[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)c.a[0][i], 2 * SUB, (int)c.w[j]);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[1][i], f.w[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)c.a[1][i], 2 * SUB, (int)c.w[j]);
    }
}

// One LDS read of the ring's per-sub-step schedule: item R < 2 WM + WN is a
// fragment of sub-step SUB (backbone rows, residual rows, then weight
// columns); the next 2 WM + WN items (SUB = 0 only) are the scale dwords in
// the same order.
template <class C, int SUB, int R>
__device__ __forceinline__ void read_item(const uint8_t* st, Frags<C>& f, Scales<C>& c, int wm, int wn, int lr,
                                          int lh) {
  constexpr int kF = 2 * C::WM + C::WN;
  if constexpr (R < 2 * C::WM) {
    constexpr int p = R / C::WM, i = R % C::WM;
    const int row = 32 * C::WM * wm + 32 * i + lr;
    f.a[p][i] = frag(st + (p ? C::kOffAr : C::kOffAs) + swz(row, 2 * SUB + lh));
  } else if constexpr (R < kF) {
    constexpr int j = R - 2 * C::WM;
    f.w[j] = frag(st + C::kOffW + swz(32 * C::WN * wn + 32 * j + lr, 2 * SUB + lh));
  } else if constexpr (SUB == 0 && R < kF + 2 * C::WM) {
    constexpr int p = (R - kF) / C::WM, i = (R - kF) % C::WM;
    const int row = 32 * C::WM * wm + 32 * i + lr;
    c.a[p][i] = *reinterpret_cast<const uint32_t*>(st + (p ? C::kOffSAr : C::kOffSAs) + 4 * row) >> (8 * lh);
  } else if constexpr (SUB == 0 && R < 2 * kF) {
    constexpr int j = R - kF - 2 * C::WM;
    c.w[j] = *reinterpret_cast<const uint32_t*>(st + C::kOffSW + 4 * (32 * C::WN * wn + 32 * j + lr)) >> (8 * lh);
  }
}

// MFMA number M of a sub-step, path-major (both paths of an accumulator are
// 2 WM WN / 2 MFMAs apart, so no MFMA waits on the one before it).
// kSkip: the wave's row blocks from `active` on hold no valid row of the tile
// (a partial last row tile of an expert segment); their MFMAs are skipped, a
// wave-uniform branch (their accumulators stay zero, and no row of theirs is
// stored).
template <class C, int SUB, int M, bool kSkip>
__device__ __forceinline__ void mfma_one(const Frags<C>& f, const Scales<C>& c, v16f (&acc)[C::WM][C::WN],
                                         int active) {
  constexpr int p = M / (C::WM * C::WN), i = (M % (C::WM * C::WN)) / C::WN, j = M % C::WN;
  if (!kSkip || i < active)
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[p][i], f.w[j], acc[i][j], 4, 4, 2 * SUB,
                                                                (int)c.a[p][i], 2 * SUB, (int)c.w[j]);
}

// ---------------------------------------------------------------------------
// Main path: buffer loads straight into a ring of LDS stages.
// ---------------------------------------------------------------------------

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (gfx9 layout): base address, no stride, `bytes` records; a
// load at an offset past `bytes` returns zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r = {(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
  return r;
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// Buffer loads that write straight into LDS: lane i of the wave stores its
// BYTES at lds + BYTES * i. They are written as inline assembly so that the
// compiler does not treat every later LDS read as dependent on them (it would
// otherwise wait for all loads in flight before each stage); completion is
// awaited explicitly with wait_vmcnt before the stage barrier. M0 carries the
// LDS base; gfx950 wants one wait state between writing M0 and the load.
__device__ __forceinline__ void buffer_to_lds16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void buffer_to_lds4(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}

template <class C>
struct RingLoader {
  i32x4 a_codes[2], w_codes;
  i32x4 s_rsrc[C::kSLoads];     // tensor of each scale run this wave loads
  uint32_t a_off[C::kAChunks];  // byte offset of this lane's A code chunk inside a stage, kOOB if absent
  uint32_t w_off[C::kWChunks];  // same for the W chunks
  uint32_t s_off[C::kSLoads];   // this lane's scale-row offset inside a stage, kOOB if absent
  bool s_is_w[C::kSLoads];      // wave-uniform: the scale run belongs to W
  int wave;                     // wave-uniform
  int nsteps;
  uint32_t a_stage_bytes, w_stage_bytes;  // scale bytes of one stage: 4 per row (codes: 64 per row)

  // Where stage s (K entries [128 s, 128 s + 128)) starts in each tensor,
  // and the LDS slot it goes to. Past the last stage every offset is moved
  // out of range: the loads keep the per-stage instruction count constant
  // and read nothing.
  struct Dest {
    uint32_t base, ka, kw, ksa, ksw;
  };
  __device__ __forceinline__ Dest dest(uint8_t* st, int s) const {
    const bool live = s < nsteps;
    Dest d;
    d.base = lds_offset(st);
    d.ka = live ? (uint32_t)s * a_stage_bytes * 16 : kOOB;  // stage start in the code arrays
    d.kw = live ? (uint32_t)s * w_stage_bytes * 16 : kOOB;
    d.ksa = live ? (uint32_t)s * a_stage_bytes : kOOB;      // and in the scale arrays
    d.ksw = live ? (uint32_t)s * w_stage_bytes : kOOB;
    return d;
  }

  // Load J of the stage (kLoads per wave): the 1 KB (16-row) chunks of the
  // two activation operands, then the weight chunks, then 64-row runs of the
  // concatenated [As | Ar | W] scale rows.
  template <int J>
  __device__ __forceinline__ void issue_j(const Dest& d) const {
    if constexpr (J < 2 * C::kAChunks) {
      constexpr int j = J / 2, p = J % 2;
      buffer_to_lds16(a_codes[p], a_off[j] + d.ka, d.base + (p ? C::kOffAr : C::kOffAs) + 1024 * (wave + C::kWaves * j));
    } else if constexpr (J < 2 * C::kAChunks + C::kWChunks) {
      constexpr int j = J - 2 * C::kAChunks;
      buffer_to_lds16(w_codes, w_off[j] + d.kw, d.base + C::kOffW + 1024 * (wave + C::kWaves * j));
    } else if constexpr (J < C::kLoads) {
      constexpr int i = J - 2 * C::kAChunks - C::kWChunks;
      buffer_to_lds4(s_rsrc[i], s_off[i] + (s_is_w[i] ? d.ksw : d.ksa), d.base + C::kOffSAs + 256 * (wave + C::kWaves * i));
    }
  }

  template <int J = 0>
  __device__ __forceinline__ void issue_all(const Dest& d) const {
    if constexpr (J < C::kLoads) {
      issue_j<J>(d);
      issue_all<J + 1>(d);
    }
  }

  // All loads of stage s into `st` at once (the ring's prologue).
  __device__ __forceinline__ void issue(uint8_t* st, int s) const { issue_all(dest(st, s)); }
};

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Barrier for the LDS ring. The vector-memory wait for the stage about to be
// read is issued separately (wait_vmcnt); a fenced __syncthreads() would wait
// for every buffer->LDS load in flight, including the stages being prefetched.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Iteration s of the ring: `cur` holds stage s, `next` stage s+1. On entry
// f0 / c hold sub-step 0 of stage s. Each half of the iteration is one MFMA
// group with the other work threaded between its MFMAs, one item after each
// MFMA, so that the MFMA pipe is fed from the first instruction after every
// wait (measured 4-10% faster than issuing the loads and LDS reads in bursts
// around the groups):
//   first half:  the sub-step 0 MFMAs of stage s, each followed by one
//                fragment read of sub-step 1 of stage s;
//   then the wait for stage s+1 and the barrier, after which the slot of
//   stage s is free (every wave holds its fragments in registers);
//   second half: the sub-step 1 MFMAs of stage s, each followed by one load
//                of stage s+kRing into the freed slot and one LDS read of
//                stage s+1 (fragments of sub-step 0, then the scales).
// Every iteration has the same shape (batches past the last stage are issued
// with out-of-range offsets and read nothing), so the vmcnt bound is a
// constant and no branch splits the MFMA groups from the barrier.
template <class C, int M, bool kSkip>
__device__ __forceinline__ void ring_first_half(const Frags<C>& f0, const Scales<C>& c, v16f (&acc)[C::WM][C::WN],
                                                const uint8_t* cur, Frags<C>& f1, Scales<C>& unused, int wm, int wn,
                                                int lr, int lh, int active) {
  if constexpr (M < 2 * C::WM * C::WN) {
    mfma_one<C, 0, M, kSkip>(f0, c, acc, active);
    read_item<C, 1, M>(cur, f1, unused, wm, wn, lr, lh);
    __builtin_amdgcn_sched_barrier(0);
    ring_first_half<C, M + 1, kSkip>(f0, c, acc, cur, f1, unused, wm, wn, lr, lh, active);
  }
}

template <class C, int M, bool kSkip>
__device__ __forceinline__ void ring_second_half(const Frags<C>& f1, const Scales<C>& c, v16f (&acc)[C::WM][C::WN],
                                                 const RingLoader<C>& ld, const typename RingLoader<C>::Dest& d,
                                                 const uint8_t* next, Frags<C>& f0, Scales<C>& cn, int wm, int wn,
                                                 int lr, int lh, int active) {
  constexpr int kMfma = 2 * C::WM * C::WN;
  constexpr int kItems = 2 * (2 * C::WM + C::WN);
  if constexpr (M < kMfma || M < C::kLoads || M < kItems) {
    if constexpr (M < kMfma) mfma_one<C, 1, M, kSkip>(f1, c, acc, active);
    ld.template issue_j<M>(d);
    read_item<C, 0, M>(next, f0, cn, wm, wn, lr, lh);
    __builtin_amdgcn_sched_barrier(0);
    ring_second_half<C, M + 1, kSkip>(f1, c, acc, ld, d, next, f0, cn, wm, wn, lr, lh, active);
  }
}

template <class C, bool kSkip>
__device__ __forceinline__ void ring_iter(const RingLoader<C>& ld, uint8_t* cur, const uint8_t* next, int s,
                                          Frags<C>& f0, Frags<C>& f1, Scales<C>& c, Scales<C>& cn,
                                          v16f (&acc)[C::WM][C::WN], int wm, int wn, int lr, int lh, int active) {
  static_assert(2 * C::WM + C::WN <= 2 * C::WM * C::WN, "every fragment read of sub-step 1 follows an MFMA");
  // a wave issuing its MFMA group gets issue priority over a wave of the
  // other workgroup on the SIMD that is loading or waiting
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  ring_first_half<C, 0, kSkip>(f0, c, acc, cur, f1, cn, wm, wn, lr, lh, active);
  __builtin_amdgcn_s_setprio(0);
  wait_vmcnt<(C::kRing - 2) * C::kLoads>();  // batch s+1 landed; later batches may be in flight
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const typename RingLoader<C>::Dest d = ld.dest(cur, s + C::kRing);
  __builtin_amdgcn_s_setprio(1);
  ring_second_half<C, 0, kSkip>(f1, c, acc, ld, d, next, f0, cn, wm, wn, lr, lh, active);
  __builtin_amdgcn_s_setprio(0);
  c = cn;
}

// The ring's stages sit back to back in one LDS array, kStage bytes apart.
// The loop is kept rolled (the slot is a uniform runtime index): unrolling it
// by the ring length makes the register allocator rotate fragment registers
// between copies and, at 256 accumulators, spill.
template <class C, bool kSkip = false>
__device__ __forceinline__ void mainloop_ring(const Operands& op, const TileRows& tr, const TileCols& tc, uint8_t* ring,
                                              v16f (&acc)[C::WM][C::WN], int s_begin, int s_end) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::NWM, wn = wave / C::NWM;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t G = op.nsteps;
  // row blocks of this wave with at least one valid row (all of them unless kSkip)
  const int64_t first_row = 32 * C::WM * wm;
  const int active = __builtin_amdgcn_readfirstlane(
      !kSkip ? C::WM
      : tr.rows_valid <= first_row ? 0
      : (int)min<int64_t>((tr.rows_valid - first_row + 31) / 32, C::WM));

  RingLoader<C> ld;
  ld.wave = wave;
  ld.a_codes[0] = make_rsrc(op.a_codes[0], op.a_rows_total * G * kRowBytes);
  ld.a_codes[1] = make_rsrc(op.a_codes[1], op.a_rows_total * G * kRowBytes);
  ld.w_codes = make_rsrc(op.w_codes, op.O * G * kRowBytes);
  const i32x4 as_rsrc0 = make_rsrc(op.a_scales[0], op.a_rows_total * G * 4);
  const i32x4 as_rsrc1 = make_rsrc(op.a_scales[1], op.a_rows_total * G * 4);
  const i32x4 ws_rsrc = make_rsrc(op.w_scales, op.O * G * 4);
  ld.a_stage_bytes = (uint32_t)(op.a_rows_total * 4);
  ld.w_stage_bytes = (uint32_t)(op.O * 4);
  // The LDS chunk position a lane fills is fixed (lane * 16 inside its 1 KB
  // chunk); pick the global 16-byte chunk that belongs there after the swizzle.
#pragma unroll
  for (int j = 0; j < C::kAChunks; ++j) {
    const int row = 16 * (wave + C::kWaves * j) + (lane >> 2);
    const int part = (lane & 3) ^ swz_part(row);
    const int64_t src = tr.src(row);
    ld.a_off[j] = src >= 0 ? (uint32_t)(src * kRowBytes + part * 16) : kOOB;
  }
#pragma unroll
  for (int j = 0; j < C::kWChunks; ++j) {
    const int row = 16 * (wave + C::kWaves * j) + (lane >> 2);
    const int part = (lane & 3) ^ swz_part(row);
    const int64_t o = tc.w_row(row);
    ld.w_off[j] = o < op.O ? (uint32_t)(o * kRowBytes + part * 16) : kOOB;
  }
  // scale runs: 64-row run q of [backbone rows | residual rows | weight rows]
#pragma unroll
  for (int i = 0; i < C::kSLoads; ++i) {
    const int q = wave + C::kWaves * i;
    constexpr int qa = C::kARunRows / 64;
    if (q >= C::kSRuns) {  // spare instruction: reads nothing, lands in the trash area
      ld.s_rsrc[i] = ws_rsrc;
      ld.s_off[i] = kOOB;
      ld.s_is_w[i] = true;
    } else if (q < 2 * qa) {
      const int64_t src = tr.src(64 * (q % qa) + lane);
      ld.s_rsrc[i] = q < qa ? as_rsrc0 : as_rsrc1;
      ld.s_off[i] = src >= 0 ? (uint32_t)(src * 4) : kOOB;
      ld.s_is_w[i] = false;
    } else {
      const int64_t o = tc.w_row(64 * (q - 2 * qa) + lane);
      ld.s_rsrc[i] = ws_rsrc;
      ld.s_off[i] = o < op.O ? (uint32_t)(o * 4) : kOOB;
      ld.s_is_w[i] = true;
    }
  }

  // stages [s_begin, s_end) of K (a split-K slice, or all of K)
  ld.nsteps = s_end;
#pragma unroll
  for (int b = 0; b < C::kRing; ++b) ld.issue(ring + b * C::kStage, s_begin + b);
  wait_vmcnt<(C::kRing - 1) * C::kLoads>();  // the first batch landed
  ring_barrier();
  Frags<C> f0, f1;
  Scales<C> c, cn;
  read_scales<C>(ring, c, wm, wn, lr, lh);
  read_frags<C, 0>(ring, f0, wm, wn, lr, lh);
  int slot = 0;
#pragma unroll 1
  for (int s = s_begin; s < s_end; ++s) {
    const int nslot = slot + 1 == C::kRing ? 0 : slot + 1;
    ring_iter<C, kSkip>(ld, ring + slot * C::kStage, ring + nslot * C::kStage, s, f0, f1, c, cn, acc, wm, wn, lr, lh,
                        active);
    slot = nslot;
  }
  wait_vmcnt<0>();  // drain the trailing out-of-range batches before the LDS is reused
}

// ---------------------------------------------------------------------------
// General path (K % 128 != 0): two LDS stages staged through registers, on
// the 128 x 256 tile.
// ---------------------------------------------------------------------------

using RegTile = SmallTile;

struct Prefetch {
  uint4 a[2][2];  // [path][chunk]
  uint4 w[4];
  uint32_t sa;    // scale dword of one A row of one path
  uint32_t sw;    // scale dword of one W row
};

// The scale dword of (stage s, row) in the stage-major layout; bytes of a
// last, partial stage past the row's blocks are masked to zero (their codes
// are not read either).
__device__ __forceinline__ uint32_t load_scales4(const uint8_t* scales, int64_t row, int64_t rows, int64_t s,
                                                 int64_t kblocks) {
  uint32_t v = *reinterpret_cast<const uint32_t*>(scales + s * rows * 4 + row * 4);
  const int64_t valid = kblocks - 4 * s;
  if (valid < 4) v &= (1u << (8 * valid)) - 1u;
  return v;
}

__device__ __forceinline__ void load_stage_regs(Prefetch& pf, const Operands& op, int s, int tid,
                                                const int64_t (&a_src)[2], int64_t a_src_scale,
                                                const int64_t (&w_row)[4], int64_t w_row_scale) {
  const int part = tid & 3;
  // block `part` of the stage exists (the padding blocks of a last, partial
  // stage are zero in a well-formed tensor; they are not read)
  const bool col_ok = 4 * (int64_t)s + part < (op.K >> 5);
  const int64_t a_stage = (int64_t)s * op.a_rows_total * kRowBytes + part * 16;
  const int64_t w_stage = (int64_t)s * op.O * kRowBytes + part * 16;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t r = a_src[c];
    const bool ok = r >= 0 && col_ok;
    const int64_t off = ok ? a_stage + r * kRowBytes : 0;
    const uint4 v0 = *reinterpret_cast<const uint4*>(op.a_codes[0] + off);
    const uint4 v1 = *reinterpret_cast<const uint4*>(op.a_codes[1] + off);
    pf.a[0][c] = ok ? v0 : make_uint4(0, 0, 0, 0);
    pf.a[1][c] = ok ? v1 : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t r = w_row[c];
    const bool ok = r >= 0 && col_ok;
    const uint4 v = *reinterpret_cast<const uint4*>(op.w_codes + (ok ? w_stage + r * kRowBytes : 0));
    pf.w[c] = ok ? v : make_uint4(0, 0, 0, 0);
  }
  const int64_t kblocks = op.K >> 5;
  const uint8_t* sbase = (tid >> 7) ? op.a_scales[1] : op.a_scales[0];
  pf.sa = a_src_scale >= 0 ? load_scales4(sbase, a_src_scale, op.a_rows_total, s, kblocks) : 0x7F7F7F7Fu;
  pf.sw = w_row_scale >= 0 ? load_scales4(op.w_scales, w_row_scale, op.O, s, kblocks) : 0x7F7F7F7Fu;
}

__device__ __forceinline__ void store_stage_regs(const Prefetch& pf, uint8_t* st, int tid) {
  const int part = tid & 3;
  const int r0 = tid >> 2;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = r0 + 64 * c;
    *reinterpret_cast<uint4*>(st + RegTile::kOffAs + swz(row, part)) = pf.a[0][c];
    *reinterpret_cast<uint4*>(st + RegTile::kOffAr + swz(row, part)) = pf.a[1][c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(st + RegTile::kOffW + swz(r0 + 64 * c, part)) = pf.w[c];
  *reinterpret_cast<uint32_t*>(st + ((tid >> 7) ? RegTile::kOffSAr : RegTile::kOffSAs) + 4 * (tid & 127)) = pf.sa;
  *reinterpret_cast<uint32_t*>(st + RegTile::kOffSW + 4 * tid) = pf.sw;
}

__device__ __forceinline__ void mainloop_regs(const Operands& op, const TileRows& tr, int64_t n0, uint8_t* buf0,
                                              uint8_t* buf1, v16f (&acc)[RegTile::WM][RegTile::WN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  int64_t a_src[2], w_row[4];
#pragma unroll
  for (int c = 0; c < 2; ++c) a_src[c] = tr.src((tid >> 2) + 64 * c);
  const int64_t a_src_scale = tr.src(tid & 127);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t o = n0 + (tid >> 2) + 64 * c;
    w_row[c] = o < op.O ? o : -1;
  }
  const int64_t os = n0 + tid;
  const int64_t w_row_scale = os < op.O ? os : -1;

  Prefetch pf;
  load_stage_regs(pf, op, 0, tid, a_src, a_src_scale, w_row, w_row_scale);
  store_stage_regs(pf, buf0, tid);
  __syncthreads();
  for (int s = 0; s < op.nsteps; ++s) {
    const uint8_t* cur = (s & 1) ? buf1 : buf0;
    const bool more = s + 1 < op.nsteps;
    if (more) load_stage_regs(pf, op, s + 1, tid, a_src, a_src_scale, w_row, w_row_scale);
    Frags<RegTile> f;
    Scales<RegTile> c;
    read_scales<RegTile>(cur, c, wm, wn, lr, lh);
    read_frags<RegTile, 0>(cur, f, wm, wn, lr, lh);
    mfma_sub<RegTile, 0>(f, c, acc);
    read_frags<RegTile, 1>(cur, f, wm, wn, lr, lh);
    mfma_sub<RegTile, 1>(f, c, acc);
    if (more) store_stage_regs(pf, (s & 1) ? buf0 : buf1, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

template <class C>
__device__ __forceinline__ void zero_acc(v16f (&acc)[C::WM][C::WN]) {
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = v16f{};
}

// Store the tile: output row m0 + r (r < rows_valid) of y with leading
// dimension ldy. Each MFMA tile is stored on its own (the scheduling barrier
// keeps the compiler from moving every accumulator into VGPRs at once); a
// tile that lies wholly inside Y skips the per-element bounds checks.
template <class C>
__device__ __forceinline__ void store_tile(const v16f (&acc)[C::WM][C::WN], float* __restrict__ y, int64_t ldy,
                                           int64_t m0, int64_t rows_valid, int64_t n0, int64_t O) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::NWM, wn = wave / C::NWM;
  const int lr = lane & 31, lh = lane >> 5;
  const bool full = rows_valid == C::BM && n0 + C::BN <= O;
  float* base = y + (m0 + 32 * C::WM * wm + 4 * lh) * ldy + n0 + 32 * C::WN * wn + lr;
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          base[(32 * i + 8 * (r >> 2) + (r & 3)) * ldy + 32 * j] = acc[i][j][r];
      } else {
        const int64_t o = n0 + 32 * C::WN * wn + 32 * j + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 32 * C::WM * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (rr < rows_valid && o < O) y[(m0 + rr) * ldy + o] = acc[i][j][r];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Tile order. Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2; block b is remapped so that each XCD receives a contiguous
// range of tile indices. Inside a range, tiles go in groups of 4 row tiles:
// the group's column tiles are walked with the 4 row tiles innermost, so the
// tiles in flight on one XCD share 4 activation row tiles and a few weight
// column tiles (measured 2-6% faster than row tiles innermost over all rows).
struct TileIndex {
  int tm, tn;
};
// Tile t of tiles_total in walking order: groups of 4 row tiles walk the
// column tiles with the row tiles innermost.
__device__ __forceinline__ TileIndex tile_order(int tile, int tiles_m, int tiles_total) {
  constexpr int kGroup = 4;
  const int tiles_n = tiles_total / tiles_m;
  const int group = tile / (kGroup * tiles_n);
  const int first_m = group * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int in_group = tile - group * kGroup * tiles_n;
  return TileIndex{first_m + in_group % gsize, in_group / gsize};
}

// Workgroups are dispatched round-robin over the 8 XCDs: block b of a grid
// of n (n % 8 == 0) becomes item (b % 8) (n / 8) + b / 8, so that each XCD
// takes a contiguous range of items.
__device__ __forceinline__ int xcd_item(int b, int n) {
  return (n & 7) == 0 ? (b & 7) * (n >> 3) + (b >> 3) : b;
}

__device__ __forceinline__ TileIndex tile_index(int b, int tiles_m, int tiles_total) {
  return tile_order(xcd_item(b, tiles_total), tiles_m, tiles_total);
}

// LDS of the main loops: the ring's stages, or the general path's double buffer.
#define SHARQ_GEMM_LDS(C, kRingPath) \
  __shared__ __attribute__((aligned(16))) uint8_t lds[(kRingPath ? C::kRing : 2) * C::kStage];

// Plain two-path GEMM, tiles in tile_index order.
template <class C, bool kRingPath>
__global__ __launch_bounds__(C::kThreads, kRingPath ? C::kOccupancy : 1) void linear_kernel(Operands op, int64_t T, float* __restrict__ y,
                                                          int64_t ldy, int tiles_m, int tiles_total) {
  SHARQ_GEMM_LDS(C, kRingPath)
  const TileIndex ti = tile_index(blockIdx.x, tiles_m, tiles_total);
  const int tm = ti.tm, tn = ti.tn;
  TileRows tr;
  tr.m0 = (int64_t)tm * C::BM;
  tr.rows_valid = T - tr.m0 < C::BM ? T - tr.m0 : C::BM;
  tr.gather = nullptr;
  tr.src_rows = T;
  const int64_t n0 = (int64_t)tn * C::BN;
  v16f acc[C::WM][C::WN];
  zero_acc<C>(acc);
  if constexpr (kRingPath)
    mainloop_ring<C>(op, tr, TileCols{n0, 0}, lds, acc, 0, op.nsteps);
  else
    mainloop_regs(op, tr, n0, lds, lds + C::kStage, acc);
  store_tile<C>(acc, y, ldy, tr.m0, tr.rows_valid, n0, op.O);
}

// Split-K two-path GEMM for problems with too few output tiles to fill the
// GPU and a long enough K (split_plan). Item q of the S * tiles work items
// (numbered in XCD ranges) computes split q / tiles (stages [S0, S1) of K,
// S0 = split * nsteps / S) of tile q % tiles and stores its fp32 partial tile
// in partials[split] ([S][T][O]); split_reduce_kernel then sums the partials in
// split order 0, 1, ..., S-1, so the result does not depend on timing. The
// kernel boundary between the two launches makes the partials visible to
// every XCD.
template <class C>
__global__ __launch_bounds__(C::kThreads, C::kOccupancy) void linear_split_kernel(Operands op, int64_t T,
                                                                              int tiles_m, int tiles_total, int S,
                                                                              float* __restrict__ partials) {
  SHARQ_GEMM_LDS(C, true)
  // split-major items in XCD ranges: an XCD takes one or a few K slices of
  // neighbouring tiles, so each weight slice is read into one L2
  const int item = xcd_item(blockIdx.x, tiles_total * S);
  const int split = item / tiles_total;
  const TileIndex ti = tile_order(item - split * tiles_total, tiles_m, tiles_total);
  TileRows tr;
  tr.m0 = (int64_t)ti.tm * C::BM;
  tr.rows_valid = T - tr.m0 < C::BM ? T - tr.m0 : C::BM;
  tr.gather = nullptr;
  tr.src_rows = T;
  const int64_t n0 = (int64_t)ti.tn * C::BN;
  v16f acc[C::WM][C::WN];
  zero_acc<C>(acc);
  const int s0 = (int)((int64_t)split * op.nsteps / S), s1 = (int)((int64_t)(split + 1) * op.nsteps / S);
  mainloop_ring<C>(op, tr, TileCols{n0, 0}, lds, acc, s0, s1);
  store_tile<C>(acc, partials + (int64_t)split * T * op.O, op.O, tr.m0, tr.rows_valid, n0, op.O);
}

constexpr int kMaxSplits = 16;

// y[t][o] = sum over q = 0 .. S-1, in that order, of partials[q][t][o]; all
// S loads of an element are issued before the adds.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ partials, int S, int64_t T,
                                                           int64_t O, float* __restrict__ y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= T * O) return;
  const int64_t t = e / O, o = e - t * O;
  float part[kMaxSplits];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q) part[q] = q < S ? partials[(int64_t)q * T * O + e] : 0.0f;
  float v = part[0];
#pragma unroll
  for (int q = 1; q < kMaxSplits; ++q)
    if (q < S) v += part[q];
  y[t * ldy + o] = v;
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

// Tile of a grouped launch. The grid is one-dimensional over (row slot,
// column tile) pairs, column tiles innermost. With kXcdRanges the pairs are
// remapped so that each XCD (to which workgroups are dealt round-robin)
// receives a contiguous range: the column tiles of one row tile then share
// its activation rows, and the row tiles of one expert its weight tiles, in
// that XCD's L2. Without it, pair b runs on XCD b mod 8, which for 8 column
// tiles gives each XCD a fixed column slice of every weight. The row slot is
// a linear index over all (expert, row-tile) pairs, expert e holding
// ceil(count_e / BM) row tiles in expert order; the expert is found by a wave-wide prefix sum of the
// per-expert tile counts. Returns e = -1 (uniform over the workgroup) for the
// surplus indices of the grid's upper bound. Segment bounds are clamped to
// [0, P], so malformed offsets never address rows outside the output.
struct GroupedTile {
  int e, col;
  TileRows tr;
};
__device__ __forceinline__ int64_t seg_bound(const int32_t* __restrict__ seg, int e, int64_t lo, int64_t P) {
  const int64_t v = seg[e];
  return v < lo ? lo : v > P ? P : v;
}

template <class C>
__device__ __forceinline__ int expert_row_tiles(const int32_t* __restrict__ seg, int e, int E, int64_t P) {
  if (e >= E) return 0;
  const int64_t lo = seg_bound(seg, e, 0, P);
  return (int)((seg_bound(seg, e + 1, lo, P) - lo + C::BM - 1) / C::BM);
}

template <class C, bool kXcdRanges>
__device__ __forceinline__ GroupedTile grouped_tile(const int32_t* __restrict__ seg, int E, int64_t P,
                                                    const int32_t* __restrict__ a_rows, int64_t src_rows,
                                                    int tiles_n) {
  __shared__ int s_info[3];
  const int tid = threadIdx.x;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  if (tid < 64) {
    // With kXcdRanges, pass 1 counts the real tiles A; the first A (rounded
    // up to 8) workgroups take the work, so that every XCD gets an equal
    // share, XCD x the logical range [x A8 / 8, (x + 1) A8 / 8).
    const int b = blockIdx.x;
    int logical = b, target = b / tiles_n;  // slots past the last tile find no expert
    if constexpr (kXcdRanges) {
      int rows_total = 0;
      for (int e0 = 0; e0 < E; e0 += 64) {
        int tiles = expert_row_tiles<C>(seg, e0 + tid, E, P);
        for (int off = 32; off > 0; off >>= 1) tiles += __shfl_xor(tiles, off, 64);
        rows_total += tiles;
      }
      const int A = rows_total * tiles_n, A8 = (A + 7) & ~7;
      logical = b < A8 ? (b & 7) * (A8 >> 3) + (b >> 3) : A;
      target = logical < A ? logical / tiles_n : -1;
    }
    if (tid == 0) s_info[2] = logical - (logical / tiles_n) * tiles_n;
    // Pass 2: the expert holding row slot target.
    int base = 0;
    for (int e0 = 0; e0 < E && target >= 0; e0 += 64) {
      const int e = e0 + tid;
      const int tiles = expert_row_tiles<C>(seg, e, E, P);
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
  GroupedTile g;
  g.e = s_info[0];
  g.col = s_info[2];
  if (g.e >= 0) {
    const int64_t lo = seg_bound(seg, g.e, 0, P);
    g.tr.m0 = lo + (int64_t)s_info[1] * C::BM;
    const int64_t hi = seg_bound(seg, g.e + 1, lo, P);
    g.tr.rows_valid = hi - g.tr.m0 < C::BM ? hi - g.tr.m0 : C::BM;
    g.tr.gather = a_rows;
    g.tr.src_rows = src_rows;
  }
  return g;
}

// Operands of expert e: its weight within the [E][G][O][64] / [E][G][O][4] stack.
__device__ __forceinline__ void select_expert(Operands& op, int e, const uint8_t* __restrict__ w_codes_all,
                                              const uint8_t* __restrict__ w_scales_all) {
  op.w_codes = w_codes_all + (int64_t)e * op.O * kRowBytes * op.nsteps;
  op.w_scales = w_scales_all + (int64_t)e * op.O * 4 * op.nsteps;
}

// Grouped two-path GEMM over token-sorted expert segments (128 x 256 tiles);
// The grid covers tiles_n column tiles times an upper bound of row slots.
template <bool kRingPath>
__global__ __launch_bounds__(kThreads, kRingPath ? SmallTile::kOccupancy : 1) void linear_grouped_kernel(
    Operands op, const int32_t* __restrict__ a_rows, const int32_t* __restrict__ seg, int E,
    const uint8_t* __restrict__ w_codes_all, const uint8_t* __restrict__ w_scales_all, float* __restrict__ y,
    int64_t P, int tiles_n) {
  using C = SmallTile;
  SHARQ_GEMM_LDS(C, kRingPath)
  const GroupedTile g = grouped_tile<C, false>(seg, E, P, a_rows, op.a_rows_total, tiles_n);
  if (g.e < 0) return;  // uniform across the workgroup
  const int64_t n0 = (int64_t)g.col * C::BN;
  select_expert(op, g.e, w_codes_all, w_scales_all);
  v16f acc[C::WM][C::WN];
  zero_acc<C>(acc);
  if constexpr (kRingPath)
    mainloop_ring<C, true>(op, g.tr, TileCols{n0, 0}, lds, acc, 0, op.nsteps);
  else
    mainloop_regs(op, g.tr, n0, lds, lds + C::kStage, acc);
  store_tile<C>(acc, y, op.O, g.tr.m0, g.tr.rows_valid, n0, op.O);
}

// ---------------------------------------------------------------------------
// Fused gate|up projection: two-path GEMM -> silu(gate) * up -> prepare.
// ---------------------------------------------------------------------------

// Outputs of the fused epilogue: h itself and/or its prepared form (the
// activation of the down projection), each optional.
struct HOutputs {
  uint16_t* h;  // bf16 [T][I] or nullptr
  uint8_t* bb_codes;  // [I/128][T][64] or nullptr (then no prepared output)
  uint8_t* bb_scales;
  uint8_t* res_codes;
  uint8_t* res_scales;
  uint8_t* mask;  // [T][I/8] or nullptr
  int64_t T, I;
};

constexpr int kHStride = 272;  // bytes per h row in LDS: 256 + 16 keeps row starts on distinct banks

// The tile's h = bf16(silu(gate) * up) (BM rows x 128 h columns) goes
// through LDS so that each lane then owns whole 32-entry blocks of h rows:
// 4 BM (row, block) pairs, each coded by the same per-block prepare
// arithmetic as the prepare kernel. A wave's four 32-column MFMA tiles are
// gate, gate, up, up of 64 h columns (TileCols).
template <class C, int N, int M>
__device__ __forceinline__ void silu_prepare_epilogue(const v16f (&acc)[C::WM][C::WN], uint8_t* lds,
                                                      const TileRows& tr, int64_t h0, const HOutputs& out) {
  static_assert(C::WN == 4, "gate, gate, up, up column tiles per wave");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::NWM, wn = wave / C::NWM;
  const int lr = lane & 31, lh = lane >> 5;
  ring_barrier();  // every wave is done with the ring before it is overwritten
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 64 * wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * C::WM * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const uint32_t hb = bf16_rne_bits(silu_times(acc[i][j][r], acc[i][j + 2][r]));
        *reinterpret_cast<uint16_t*>(lds + row * kHStride + 2 * col) = (uint16_t)hb;
      }
    }
  __syncthreads();
  const int64_t blk0 = h0 >> 5;  // first 32-block of the tile along I
#pragma unroll
  for (int k = 0; k < (4 * C::BM + C::kThreads - 1) / C::kThreads; ++k) {
    const int p = tid + C::kThreads * k;
    const int row = p >> 2, blk = p & 3;
    if (row >= C::BM || row >= tr.rows_valid) continue;
    const int64_t t = tr.m0 + row;
    const uint4* src = reinterpret_cast<const uint4*>(lds + row * kHStride + 64 * blk);
    uint4 raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = src[q];
    if (out.h) {
      uint4* dst = reinterpret_cast<uint4*>(out.h + t * out.I + h0 + 32 * blk);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = raw[q];
    }
    if (out.bb_codes) {
      float xv[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[8 * q + 2 * e] = bf16_lo(w[e]);
          xv[8 * q + 2 * e + 1] = bf16_hi(w[e]);
        }
      }
      const PreparedBlock pb = prepare_block<N, M, false>(xv);
      const uint32_t b = (uint32_t)(blk0 + blk);
      *reinterpret_cast<uint4*>(out.bb_codes + code_offset(t, b, out.T)) = pb.c_bb;
      *reinterpret_cast<uint4*>(out.res_codes + code_offset(t, b, out.T)) = pb.c_rs;
      out.bb_scales[scale_index(t, b, out.T)] = (uint8_t)pb.e_bb;
      out.res_scales[scale_index(t, b, out.T)] = (uint8_t)pb.e_rs;
      if (out.mask) reinterpret_cast<uint32_t*>(out.mask)[t * (out.I >> 5) + b] = pb.keep;
    }
  }
}

// One 128 x 128 h tile: the two-path GEMM over the tile's 128 gate and 128 up
// weight rows, then the fused epilogue.
template <class C, int N, int M>
__global__ __launch_bounds__(C::kThreads, C::kOccupancy) void linear_silu_prepare_kernel(Operands op, HOutputs out,
                                                                                         int tiles_m,
                                                                                         int tiles_total) {
  static_assert(C::BN == 256, "one tile covers 128 h columns");
  static_assert(C::kRing * C::kStage >= C::BM * kHStride, "the h tile must fit in the ring's LDS");
  SHARQ_GEMM_LDS(C, true)
  const TileIndex ti = tile_index(blockIdx.x, tiles_m, tiles_total);
  const int tm = ti.tm, tn = ti.tn;
  TileRows tr;
  tr.m0 = (int64_t)tm * C::BM;
  tr.rows_valid = out.T - tr.m0 < C::BM ? out.T - tr.m0 : C::BM;
  tr.gather = nullptr;
  tr.src_rows = out.T;
  const int64_t h0 = (int64_t)tn * 128;
  v16f acc[C::WM][C::WN];
  zero_acc<C>(acc);
  mainloop_ring<C>(op, tr, TileCols{h0, out.I}, lds, acc, 0, op.nsteps);
  silu_prepare_epilogue<C, N, M>(acc, lds, tr, h0, out);
}

// Split-K form of the fused gate|up epilogue, for problems that the split
// plan splits (too few tiles to fill the GPU, long K). linear_split_kernel has stored the
// partials [S][T][2I] of the plain gate|up GEMM; here lane (t, b) owns the
// 32-entry h block b of row t (a wave: a 16-row band of one 128-entry stage,
// as in the prepare kernel), sums the S partials of its 32 gate and 32 up
// outputs in split order 0, 1, ..., S-1 (as split_reduce_kernel), forms
// h = bf16(silu(g) * u) (as the SiLU kernel) and codes the block with the
// per-block prepare code. The results equal linear (split-K) -> silu_mul ->
// prepare bit for bit, with neither the fp32 gate|up output nor h in HBM.
template <int N, int M>
__global__ __launch_bounds__(256) void split_reduce_silu_prepare_kernel(const float* __restrict__ partials, int S,
                                                                        HOutputs out) {
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  const uint32_t item = gid >> 6, lane = gid & 63;
  const uint32_t stages = (uint32_t)(out.I / 128);
  const uint32_t band = item / stages, g = item - band * stages;
  const int64_t t = (int64_t)band * 16 + (lane >> 2);
  const uint32_t b = g * 4 + (lane & 3);
  if (t >= out.T) return;  // per lane: no barrier follows
  const int64_t plane = out.T * 2 * out.I;
  const float* gsrc = partials + t * 2 * out.I + 32 * (int64_t)b;
  const float* usrc = gsrc + out.I;
  float gv[32], uv[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 a = reinterpret_cast<const float4*>(gsrc)[k];
    const float4 c = reinterpret_cast<const float4*>(usrc)[k];
    gv[4 * k] = a.x, gv[4 * k + 1] = a.y, gv[4 * k + 2] = a.z, gv[4 * k + 3] = a.w;
    uv[4 * k] = c.x, uv[4 * k + 1] = c.y, uv[4 * k + 2] = c.z, uv[4 * k + 3] = c.w;
  }
  for (int q = 1; q < S; ++q) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 a = reinterpret_cast<const float4*>(gsrc + q * plane)[k];
      const float4 c = reinterpret_cast<const float4*>(usrc + q * plane)[k];
      gv[4 * k] += a.x, gv[4 * k + 1] += a.y, gv[4 * k + 2] += a.z, gv[4 * k + 3] += a.w;
      uv[4 * k] += c.x, uv[4 * k + 1] += c.y, uv[4 * k + 2] += c.z, uv[4 * k + 3] += c.w;
    }
  }
  float hv[32];
  uint32_t hb[16];
#pragma unroll
  for (int k = 0; k < 32; k += 2) {
    hb[k / 2] = bf16x2_rne(silu_times(gv[k], uv[k]), silu_times(gv[k + 1], uv[k + 1]));
    hv[k] = bf16_lo(hb[k / 2]);
    hv[k + 1] = bf16_hi(hb[k / 2]);
  }
  if (out.h) {
    uint4* dst = reinterpret_cast<uint4*>(out.h + t * out.I + 32 * (int64_t)b);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(hb[4 * q], hb[4 * q + 1], hb[4 * q + 2], hb[4 * q + 3]);
  }
  if (out.bb_codes) {
    const PreparedBlock pb = prepare_block<N, M, false>(hv);
    *reinterpret_cast<uint4*>(out.bb_codes + code_offset(t, b, out.T)) = pb.c_bb;
    *reinterpret_cast<uint4*>(out.res_codes + code_offset(t, b, out.T)) = pb.c_rs;
    out.bb_scales[scale_index(t, b, out.T)] = (uint8_t)pb.e_bb;
    out.res_scales[scale_index(t, b, out.T)] = (uint8_t)pb.e_rs;
    if (out.mask) reinterpret_cast<uint32_t*>(out.mask)[t * (out.I >> 5) + b] = pb.keep;
  }
}

// Grouped form of the fused gate|up projection (mixture-of-experts layers):
// the tile of linear_grouped_kernel's row walk with the fused epilogue;
// the column tile is the 128-column h tile.
template <int N, int M>
__global__ __launch_bounds__(kThreads, SmallTile::kOccupancy) void linear_grouped_silu_prepare_kernel(
    Operands op, const int32_t* __restrict__ a_rows, const int32_t* __restrict__ seg, int E,
    const uint8_t* __restrict__ w_codes_all, const uint8_t* __restrict__ w_scales_all, HOutputs out, int tiles_n) {
  using C = SmallTile;
  static_assert(C::kRing * C::kStage >= 128 * kHStride, "the h tile must fit in the ring's LDS");
  SHARQ_GEMM_LDS(C, true)
  const GroupedTile g = grouped_tile<C, true>(seg, E, out.T, a_rows, op.a_rows_total, tiles_n);
  if (g.e < 0) return;
  const int64_t h0 = (int64_t)g.col * 128;
  select_expert(op, g.e, w_codes_all, w_scales_all);
  v16f acc[C::WM][C::WN];
  zero_acc<C>(acc);
  mainloop_ring<C, true>(op, g.tr, TileCols{h0, out.I}, lds, acc, 0, op.nsteps);
  silu_prepare_epilogue<C, N, M>(acc, lds, g.tr, h0, out);
}

Operands make_operands(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                       const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t rows,
                       int64_t O, int64_t K) {
  Operands op;
  op.a_codes[0] = bb_codes;
  op.a_codes[1] = res_codes;
  op.a_scales[0] = bb_scales;
  op.a_scales[1] = res_scales;
  op.w_codes = w_codes;
  op.w_scales = w_scales;
  op.a_rows_total = rows;
  op.K = K;
  op.O = O;
  op.nsteps = (int)((K + 127) / 128);
  return op;
}

// The ring path addresses every operand with 32-bit buffer offsets.
bool ring_path_ok(int64_t rows, int64_t O, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return K % 128 == 0 && rows * (K / 2) < lim && O * (K / 2) < lim;
}

// Problems with at least one tile per CU take the ring of 2 (which leaves LDS
// for a second workgroup per CU); below that the ring of 4. At exactly one
// tile per CU (the Llama-3.1-8B down projection) the ring of 2 measured 3%
// faster than the ring of 4.
constexpr int64_t kSmallTileMin = 256;

template <class C, bool kRingPath>
void launch_tiles(const Operands& op, int64_t T, float* y, int64_t ldy, hipStream_t stream) {
  const int tiles_m = (int)((T + C::BM - 1) / C::BM);
  const int tiles_n = (int)((op.O + C::BN - 1) / C::BN);
  const int total = tiles_m * tiles_n;
  hipLaunchKernelGGL((linear_kernel<C, kRingPath>), dim3(total), dim3(C::kThreads), 0, stream, op, T, y, ldy, tiles_m,
                     total);
}

// The tile of a problem with T rows on the ring path: 0 SmallTile (or
// DeepTile), 1 DecodeTile, 2 Decode64Tile.
int row_tile(int64_t T) { return T <= DecodeTile::BM ? 1 : T <= Decode64Tile::BM ? 2 : 0; }
int64_t row_tile_bm(int tile) {
  return tile == 1 ? DecodeTile::BM : tile == 2 ? Decode64Tile::BM : SmallTile::BM;
}

struct SplitPlan {
  int S;             // 1: no split
  int tile;          // row_tile(T)
  int tiles_m, tiles_total;
  int64_t partial_bytes;
};

// Split-K plan: the S in [1, 16] (each split over at least 4 stages, the
// partials at most 256 MB) with the smallest estimated launch time. The
// estimate was fitted to timed launches (S = 1 .. 16) of nine layer shapes
// on MI355X, T = 1 .. 1024, O x K from 1024 x 8192 to 57344 x 8192:
//  - the K loop: nsteps / S stages of c us (0.45 for the 32-row tile, 0.6
//    for the 64-row one, 0.72 for the 128-row one) while a CU runs one
//    workgroup; W = S * tiles workgroups put ceil(W / 256) on a CU, which
//    runs them two at a time at 1.7 times the time of one;
//  - no faster than streaming the weight and the activations (17/32 bytes
//    per weight entry, 17/16 per activation entry: two paths) at 6.5 TB/s;
//  - for S > 1, the partials: each split writes its fp32 tile and the
//    reduce reads them all and writes Y, (2S + 1) T O 4 bytes at an
//    effective 4 TB/s, plus 2 us for the second launch.
// Long-K layers whose tiles leave CUs idle split (the Llama-3.1-8B down
// projection at T = 384: 74 -> 34 us); wide layers that already fill the GPU
// or stream their weight at the HBM rate do not (the Llama-3.1-70B gate|up at
// T = 64: 71 us split in two, 48 us whole).
constexpr int64_t kMaxPartialBytes = (int64_t)256 << 20;

double split_cost_us(int64_t T, int64_t O, int64_t K, int tile, int64_t tiles, int64_t S) {
  const int64_t nsteps = K / 128;
  const double c = tile == 1 ? 0.45 : tile == 2 ? 0.6 : 0.72;
  const int64_t per_cu = (S * tiles + 255) / 256;
  const double crowd = per_cu <= 1 ? 1.0 : 1.7 * (double)per_cu / 2.0;
  const double loop = (double)nsteps / (double)S * c * crowd;
  const double stream = ((double)O * (double)K * 17.0 / 32.0 + (double)T * (double)K * 17.0 / 16.0) / 6.5e6;
  double t = loop > stream ? loop : stream;
  if (S > 1) t += 2.0 + (double)(2 * S + 1) * (double)T * (double)O * 4.0 / 4.0e6;
  return t;
}

SplitPlan split_plan(int64_t T, int64_t O, int64_t K) {
  SplitPlan p{1, 0, 0, 0, 0};
  if (T <= 0 || O <= 0 || T * O >= ((int64_t)1 << 31) || !ring_path_ok(T, O, K)) return p;
  p.tile = row_tile(T);
  const int64_t bm = row_tile_bm(p.tile);
  p.tiles_m = (int)((T + bm - 1) / bm);
  p.tiles_total = p.tiles_m * (int)((O + SmallTile::BN - 1) / SmallTile::BN);
  const int64_t s_max = K / 128 / 4 < kMaxSplits ? K / 128 / 4 : kMaxSplits;
  int64_t S = 1;
  double best = split_cost_us(T, O, K, p.tile, p.tiles_total, 1);
  for (int64_t s = 2; s <= s_max && s * T * O * 4 <= kMaxPartialBytes; ++s) {
    const double c = split_cost_us(T, O, K, p.tile, p.tiles_total, s);
    if (c < best) best = c, S = s;
  }
  if (S < 2) return p;
  p.S = (int)S;
  p.partial_bytes = S * T * O * 4;
  return p;
}

void launch_split(const SplitPlan& p, const Operands& op, int64_t T, float* partials, hipStream_t stream) {
  if (p.tile == 1)
    hipLaunchKernelGGL((linear_split_kernel<DecodeTile>), dim3(p.tiles_total * p.S), dim3(DecodeTile::kThreads), 0,
                       stream, op, T, p.tiles_m, p.tiles_total, p.S, partials);
  else if (p.tile == 2)
    hipLaunchKernelGGL((linear_split_kernel<Decode64Tile>), dim3(p.tiles_total * p.S), dim3(Decode64Tile::kThreads),
                       0, stream, op, T, p.tiles_m, p.tiles_total, p.S, partials);
  else
    hipLaunchKernelGGL((linear_split_kernel<SmallTile>), dim3(p.tiles_total * p.S), dim3(SmallTile::kThreads), 0,
                       stream, op, T, p.tiles_m, p.tiles_total, p.S, partials);
}

}  // namespace

int64_t linear_workspace_bytes(int64_t T, int64_t O, int64_t K) {
  const SplitPlan p = split_plan(T, O, K);
  return p.S > 1 ? p.partial_bytes : 0;
}

int64_t linear_silu_prepare_workspace_bytes(int64_t T, int64_t I, int64_t K) {
  const SplitPlan p = split_plan(T, 2 * I, K);
  return p.S > 1 ? p.partial_bytes : 0;
}

hipError_t launch_linear_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                            const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T,
                            int64_t O, int64_t K, float* y, int64_t ldy, void* workspace, int64_t workspace_bytes,
                            hipStream_t stream) {
  const SplitPlan p = split_plan(T, O, K);
  if (p.S < 2 || !workspace || workspace_bytes < p.partial_bytes)
    return launch_linear(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K, y, ldy, stream);
  const Operands op = make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K);
  float* partials = static_cast<float*>(workspace);
  launch_split(p, op, T, partials, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((T * O + 255) / 256)), dim3(256), 0, stream, partials,
                     p.S, T, O, y, ldy);
  return hipGetLastError();
}

hipError_t launch_linear(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  const Operands op = make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K);
  const int64_t tiles = ((T + SmallTile::BM - 1) / SmallTile::BM) * ((O + SmallTile::BN - 1) / SmallTile::BN);
  if (!ring_path_ok(T, O, K))
    launch_tiles<SmallTile, false>(op, T, y, ldy, stream);
  else if (row_tile(T) == 1)
    launch_tiles<DecodeTile, true>(op, T, y, ldy, stream);
  else if (row_tile(T) == 2)
    launch_tiles<Decode64Tile, true>(op, T, y, ldy, stream);
  else if (tiles >= kSmallTileMin)
    launch_tiles<SmallTile, true>(op, T, y, ldy, stream);
  else
    launch_tiles<DeepTile, true>(op, T, y, ldy, stream);
  return hipGetLastError();
}

hipError_t launch_linear_grouped(const uint8_t* bb_codes, const uint8_t* bb_scales,
                                 const uint8_t* res_codes, const uint8_t* res_scales,
                                 const int32_t* a_rows, const int32_t* seg_offsets, int32_t E,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t O,
                                 int64_t K, float* y, int64_t a_rows_total, hipStream_t stream) {
  const Operands op =
      make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, a_rows_total, O, K);
  // every expert contributes ceil(count / 128) row tiles: at most P/128 + E in total
  const int64_t tiles_m_bound = (P + SmallTile::BM - 1) / SmallTile::BM + E;
  const int tiles_n = (int)((O + SmallTile::BN - 1) / SmallTile::BN);
  const int total = (int)(tiles_n * tiles_m_bound);
  const dim3 grid((unsigned)total);
  if (ring_path_ok(a_rows_total, O, K))
    hipLaunchKernelGGL(linear_grouped_kernel<true>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets, E,
                       w_codes, w_scales, y, P, tiles_n);
  else
    hipLaunchKernelGGL(linear_grouped_kernel<false>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets, E,
                       w_codes, w_scales, y, P, tiles_n);
  return hipGetLastError();
}

hipError_t launch_linear_silu_prepare_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                         int64_t T, int64_t I, int64_t K, int n, int m, uint16_t* h,
                                         uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                         uint8_t* h_res_scales, uint8_t* h_mask, void* workspace,
                                         int64_t workspace_bytes, hipStream_t stream) {
  const SplitPlan p = split_plan(T, 2 * I, K);
  if (p.S < 2 || !workspace || workspace_bytes < p.partial_bytes)
    return launch_linear_silu_prepare(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, I, K, n, m, h,
                                      h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask, stream);
  const Operands op = make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, 2 * I, K);
  float* partials = static_cast<float*>(workspace);
  launch_split(p, op, T, partials, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const HOutputs out{h, h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask, T, I};
  const uint64_t lanes = (uint64_t)((T + 15) / 16) * (uint64_t)(I / 128) * 64;
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (n == 2 && m == 4)
    hipLaunchKernelGGL((split_reduce_silu_prepare_kernel<2, 4>), grid, dim3(256), 0, stream, partials, p.S, out);
  else
    hipLaunchKernelGGL((split_reduce_silu_prepare_kernel<8, 16>), grid, dim3(256), 0, stream, partials, p.S, out);
  return hipGetLastError();
}

hipError_t launch_linear_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                      const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                      int64_t T, int64_t I, int64_t K, int n, int m, uint16_t* h,
                                      uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                      uint8_t* h_res_scales, uint8_t* h_mask, hipStream_t stream) {
  const Operands op = make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, 2 * I, K);
  const HOutputs out{h, h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask, T, I};
  const int tile = row_tile(T);
  const int64_t bm = row_tile_bm(tile);
  const int tiles_m = (int)((T + bm - 1) / bm);
  const int total = tiles_m * (int)(I / 128);
  const bool two = total >= kSmallTileMin;
#define SHARQ_FUSED(C, NN, MM)                                                                                       \
  hipLaunchKernelGGL((linear_silu_prepare_kernel<C, NN, MM>), dim3(total), dim3(C::kThreads), 0, stream, op, out, \
                     tiles_m, total)
#define SHARQ_FUSED_NM(NN, MM)                        \
  if (tile == 1) SHARQ_FUSED(DecodeTile, NN, MM);     \
  else if (tile == 2) SHARQ_FUSED(Decode64Tile, NN, MM); \
  else if (two) SHARQ_FUSED(SmallTile, NN, MM);       \
  else SHARQ_FUSED(DeepTile, NN, MM)
  if (n == 2 && m == 4) {
    SHARQ_FUSED_NM(2, 4);
  } else {
    SHARQ_FUSED_NM(8, 16);
  }
#undef SHARQ_FUSED_NM
#undef SHARQ_FUSED
  return hipGetLastError();
}

hipError_t launch_linear_grouped_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales,
                                              const uint8_t* res_codes, const uint8_t* res_scales,
                                              const int32_t* a_rows, const int32_t* seg_offsets, int32_t E,
                                              const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t I,
                                              int64_t K, int64_t a_rows_total, int n, int m, uint16_t* h,
                                              uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                              uint8_t* h_res_scales, uint8_t* h_mask, hipStream_t stream) {
  const Operands op =
      make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, a_rows_total, 2 * I, K);
  const HOutputs out{h, h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask, P, I};
  const int64_t tiles_m_bound = (P + SmallTile::BM - 1) / SmallTile::BM + E;
  const int tiles_n = (int)(I / 128);
  const int total = (int)(tiles_n * tiles_m_bound);
  const dim3 grid((unsigned)total);
  if (n == 2 && m == 4)
    hipLaunchKernelGGL((linear_grouped_silu_prepare_kernel<2, 4>), grid, dim3(kThreads), 0, stream, op, a_rows,
                       seg_offsets, E, w_codes, w_scales, out, tiles_n);
  else
    hipLaunchKernelGGL((linear_grouped_silu_prepare_kernel<8, 16>), grid, dim3(kThreads), 0, stream, op, a_rows,
                       seg_offsets, E, w_codes, w_scales, out, tiles_n);
  return hipGetLastError();
}

}  // namespace sharq
