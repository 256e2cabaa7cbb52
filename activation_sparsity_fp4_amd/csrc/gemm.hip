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
// per row per operand; with the stage-major layout of sharq_device.h one stage
// of a tile is one contiguous run of every operand). A stage holds the backbone tile, the residual tile, the
// weight tile and their scales (34 KB of LDS).
//
// Main path (K % 128 == 0): a ring of 4 LDS stages filled by buffer loads that
// write straight into LDS (no register staging); four stages are in flight
// ahead of the MFMAs, rows past the end of a matrix read as zero through the
// buffer bounds check, and one barrier per stage recycles a slot as soon as
// every wave holds that stage's fragments in registers. General
// path (any K % 32 == 0): 2 LDS stages filled through registers.
//
// LDS rows are 64 bytes; the 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 2) & 3), which keeps the rows read by one MFMA fragment on
// distinct banks of the 64-bank LDS.
//
// Codes and scales are stored stage-major (sharq_device.h): one stage of a
// 128-row tile is a contiguous 8 KB run of codes and a 512-byte run of
// scales, so every load uses whole cache lines.
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
constexpr int kRing = 4;                  // LDS stages of the main path
constexpr int kLoadsPerStage = 10;        // buffer->LDS instructions per wave per stage
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every bound: reads as 0

// LDS chunk swizzle. gfx950 LDS has 64 four-byte banks; a ds_read_b128 of an
// MFMA fragment serves 16 lanes (16 consecutive rows, one 16-byte chunk each)
// per pass, and rows r and r + 4 start on the same bank. XOR-ing the chunk
// index with bits 2..3 of the row spreads those 16 rows over all 64 banks
// (measured: zero SQ_LDS_BANK_CONFLICT cycles).
__device__ __forceinline__ int swz_part(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz(int row, int part) {
  return row * kRowBytes + ((part ^ swz_part(row)) << 4);
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

// All MFMAs of one 128-entry stage held in LDS at `st`.
__device__ __forceinline__ void compute_stage(const uint8_t* st, v16f (&acc)[2][4], int wm, int wn, int lr,
                                              int lh) {
  uint32_t sa[2][2], sw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 64 * wm + 32 * i + lr;
    sa[0][i] = *reinterpret_cast<const uint32_t*>(st + kOffSAs + 4 * row) >> (8 * lh);
    sa[1][i] = *reinterpret_cast<const uint32_t*>(st + kOffSAr + 4 * row) >> (8 * lh);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    sw[j] = *reinterpret_cast<const uint32_t*>(st + kOffSW + 4 * (128 * wn + 32 * j + lr)) >> (8 * lh);
  compute_sub<0>(st, acc, wm, wn, lr, lh, sa, sw);
  compute_sub<1>(st, acc, wm, wn, lr, lh, sa, sw);
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

// Row sources of one output tile: which activation row feeds tile row r, or -1.
struct TileRows {
  int64_t m0;          // first output row of the tile
  int64_t rows_valid;  // output rows of the tile that exist (<= kBM)
  const int32_t* gather;  // activation row of each output row, or nullptr (identity)
  __device__ __forceinline__ int64_t src(int r) const {
    if (r >= rows_valid) return -1;
    const int64_t p = m0 + r;
    return gather ? (int64_t)gather[p] : p;
  }
};

// ---------------------------------------------------------------------------
// Main path: buffer loads straight into a 4-stage LDS ring.
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

struct RingLoader {
  i32x4 a_codes[2], a_scales[2], w_codes, w_scales;
  uint32_t a_off[2];   // byte offset of this lane's A code chunk inside a stage (chunks j = 0, 1), kOOB if absent
  uint32_t w_off[4];   // same for the 4 W chunks
  uint32_t s_off[2];   // scale-row byte offsets for this wave's two scale instructions
  int wave;            // wave-uniform
  int nsteps;
  uint32_t a_stage_bytes, w_stage_bytes;  // scale bytes of one stage: 4 per row (codes: 64 per row)

  // Issue the 10 loads of stage s (K entries [128 s, 128 s + 128)) into `st`.
  // Past the last stage every offset is moved out of range: the loads keep
  // the per-stage instruction count constant and read nothing.
  __device__ __forceinline__ void issue(uint8_t* st, int s) const {
    const uint32_t base = lds_offset(st);
    const bool live = s < nsteps;
    const uint32_t ka = live ? (uint32_t)s * a_stage_bytes * 16 : kOOB;  // stage start in the code arrays
    const uint32_t kw = live ? (uint32_t)s * w_stage_bytes * 16 : kOOB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = wave + 4 * j;  // 1 KB chunk inside the 8 KB A tile
      buffer_to_lds16(a_codes[0], a_off[j] + ka, base + kOffAs + 1024 * chunk);
      buffer_to_lds16(a_codes[1], a_off[j] + ka, base + kOffAr + 1024 * chunk);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = wave + 4 * j;  // 1 KB chunk inside the 16 KB W tile
      buffer_to_lds16(w_codes, w_off[j] + kw, base + kOffW + 1024 * chunk);
    }
    const uint32_t ksa = live ? (uint32_t)s * a_stage_bytes : kOOB;
    const uint32_t ksw = live ? (uint32_t)s * w_stage_bytes : kOOB;
    // scale rows: waves 0,1 -> backbone rows 64w..; waves 2,3 -> residual rows; then W rows 64w..
    const i32x4 ars = wave < 2 ? a_scales[0] : a_scales[1];
    const uint32_t aoff = (wave < 2 ? kOffSAs : kOffSAr) + 256 * (wave & 1);
    buffer_to_lds4(ars, s_off[0] + ksa, base + aoff);
    buffer_to_lds4(w_scales, s_off[1] + ksw, base + kOffSW + 256 * wave);
  }
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

// Each ring stage is its own __shared__ object so that the compiler's wait
// insertion can tell a read of one stage from the loads still filling another.
struct RingStages {
  uint8_t* st[kRing];
};

// Fragments and scale dwords of one 64-entry sub-step, held in registers.
struct Frags {
  v8i a[2][2];  // [path][row block]
  v8i w[4];
};
struct Scales {
  uint32_t a[2][2];  // [path][row block]
  uint32_t w[4];
};

template <int SUB>
__device__ __forceinline__ void read_frags(const uint8_t* st, Frags& f, int wm, int wn, int lr, int lh) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 64 * wm + 32 * i + lr;
    f.a[0][i] = frag(st + kOffAs + swz(row, 2 * SUB + lh));
    f.a[1][i] = frag(st + kOffAr + swz(row, 2 * SUB + lh));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) f.w[j] = frag(st + kOffW + swz(128 * wn + 32 * j + lr, 2 * SUB + lh));
}

__device__ __forceinline__ void read_scales(const uint8_t* st, Scales& c, int wm, int wn, int lr, int lh) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 64 * wm + 32 * i + lr;
    c.a[0][i] = *reinterpret_cast<const uint32_t*>(st + kOffSAs + 4 * row) >> (8 * lh);
    c.a[1][i] = *reinterpret_cast<const uint32_t*>(st + kOffSAr + 4 * row) >> (8 * lh);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    c.w[j] = *reinterpret_cast<const uint32_t*>(st + kOffSW + 4 * (128 * wn + 32 * j + lr)) >> (8 * lh);
}

template <int SUB>
__device__ __forceinline__ void mfma_sub(const Frags& f, const Scales& c, v16f (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[0][i], f.w[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)c.a[0][i], 2 * SUB, (int)c.w[j]);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[1][i], f.w[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)c.a[1][i], 2 * SUB, (int)c.w[j]);
    }
}

// Iteration s of the ring (slot I = s % 4). On entry f0 / c hold sub-step 0
// of stage s. The sub-step 1 reads are issued before the sub-step 0 MFMAs;
// the barrier that makes stage s+1 visible sits between the two MFMA groups,
// and the sub-step 0 reads of stage s+1 are issued before the sub-step 1
// MFMAs, so LDS latency hides behind 16 MFMAs each time. Once every wave has
// its stage-s fragments in registers (the barrier waits on lgkmcnt), slot I
// is refilled with stage s+4: four stages are in flight. Every iteration has
// the same shape (batches past the last stage are issued with out-of-range
// offsets and read nothing), so the vmcnt bound is a constant and no branch
// splits the MFMA groups from the barrier.
template <int I>
__device__ __forceinline__ void ring_iter(const RingLoader& ld, const RingStages& rs, int s, Frags& f0, Frags& f1,
                                          Scales& c, Scales& cn, v16f (&acc)[2][4], int wm, int wn, int lr, int lh) {
  read_frags<1>(rs.st[I], f1, wm, wn, lr, lh);
  mfma_sub<0>(f0, c, acc);
  // schedule: the 8 fragment reads first, then the 16 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<2 * kLoadsPerStage>();  // batch s+1 landed; s+2, s+3 may be in flight
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  ld.issue(rs.st[I], s + kRing);
  read_scales(rs.st[(I + 1) % kRing], cn, wm, wn, lr, lh);
  read_frags<0>(rs.st[(I + 1) % kRing], f0, wm, wn, lr, lh);
  mfma_sub<1>(f1, c, acc);
  // schedule: all LDS reads of stage s+1 first, then the 16 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  __builtin_amdgcn_sched_barrier(0);
  c = cn;
}

__device__ __forceinline__ void mainloop_ring(const Operands& op, const TileRows& tr, int64_t n0,
                                              const RingStages& rs, v16f (&acc)[2][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t G = op.nsteps;

  RingLoader ld;
  ld.wave = wave;
  ld.a_codes[0] = make_rsrc(op.a_codes[0], op.a_rows_total * G * kRowBytes);
  ld.a_codes[1] = make_rsrc(op.a_codes[1], op.a_rows_total * G * kRowBytes);
  ld.a_scales[0] = make_rsrc(op.a_scales[0], op.a_rows_total * G * 4);
  ld.a_scales[1] = make_rsrc(op.a_scales[1], op.a_rows_total * G * 4);
  ld.w_codes = make_rsrc(op.w_codes, op.O * G * kRowBytes);
  ld.w_scales = make_rsrc(op.w_scales, op.O * G * 4);
  ld.a_stage_bytes = (uint32_t)(op.a_rows_total * 4);
  ld.w_stage_bytes = (uint32_t)(op.O * 4);
  // The LDS chunk position a lane fills is fixed (lane * 16 inside its 1 KB
  // chunk); pick the global 16-byte chunk that belongs there after the swizzle.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (wave + 4 * j) + (lane >> 2);
    const int part = (lane & 3) ^ swz_part(row);
    const int64_t src = tr.src(row);
    ld.a_off[j] = src >= 0 ? (uint32_t)(src * kRowBytes + part * 16) : kOOB;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * (wave + 4 * j) + (lane >> 2);
    const int part = (lane & 3) ^ swz_part(row);
    const int64_t o = n0 + row;
    ld.w_off[j] = o < op.O ? (uint32_t)(o * kRowBytes + part * 16) : kOOB;
  }
  {
    const int64_t src = tr.src(64 * (wave & 1) + lane);
    ld.s_off[0] = src >= 0 ? (uint32_t)(src * 4) : kOOB;
    const int64_t o = n0 + 64 * wave + lane;
    ld.s_off[1] = o < op.O ? (uint32_t)(o * 4) : kOOB;
  }

  const int nsteps = op.nsteps;
  ld.nsteps = nsteps;
  static_assert(kRing == 4, "the iteration sequence below is unrolled for 4 stages");
#pragma unroll
  for (int b = 0; b < kRing; ++b) ld.issue(rs.st[b], b);
  wait_vmcnt<3 * kLoadsPerStage>();  // batch 0 landed
  ring_barrier();
  Frags f0, f1;
  Scales c, cn;
  read_scales(rs.st[0], c, wm, wn, lr, lh);
  read_frags<0>(rs.st[0], f0, wm, wn, lr, lh);
  for (int s = 0; s < nsteps; s += kRing) {
    ring_iter<0>(ld, rs, s, f0, f1, c, cn, acc, wm, wn, lr, lh);
    if (s + 1 < nsteps) ring_iter<1>(ld, rs, s + 1, f0, f1, c, cn, acc, wm, wn, lr, lh);
    if (s + 2 < nsteps) ring_iter<2>(ld, rs, s + 2, f0, f1, c, cn, acc, wm, wn, lr, lh);
    if (s + 3 < nsteps) ring_iter<3>(ld, rs, s + 3, f0, f1, c, cn, acc, wm, wn, lr, lh);
  }
  wait_vmcnt<0>();  // drain the trailing out-of-range batches before the LDS is reused
}

// ---------------------------------------------------------------------------
// General path (K % 128 != 0): two LDS stages staged through registers.
// ---------------------------------------------------------------------------

struct Prefetch {
  uint4 a[2][2];  // [path][chunk]
  uint4 w[4];
  uint32_t sa;    // scale dword of one A row of one path
  uint32_t sw;    // scale dword of one W row
};

// The scale dword of (stage s, row) in the stage-major layout; bytes of a
// last, partial stage past the row's blocks are masked to zero (their codes
// are zero too).
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
    *reinterpret_cast<uint4*>(st + kOffAs + swz(row, part)) = pf.a[0][c];
    *reinterpret_cast<uint4*>(st + kOffAr + swz(row, part)) = pf.a[1][c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(st + kOffW + swz(r0 + 64 * c, part)) = pf.w[c];
  *reinterpret_cast<uint32_t*>(st + ((tid >> 7) ? kOffSAr : kOffSAs) + 4 * (tid & 127)) = pf.sa;
  *reinterpret_cast<uint32_t*>(st + kOffSW + 4 * tid) = pf.sw;
}

__device__ __forceinline__ void mainloop_regs(const Operands& op, const TileRows& tr, int64_t n0, uint8_t* buf0,
                                              uint8_t* buf1, v16f (&acc)[2][4]) {
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
    compute_stage(cur, acc, wm, wn, lr, lh);
    if (more) store_stage_regs(pf, (s & 1) ? buf0 : buf1, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

__device__ __forceinline__ void zero_acc(v16f (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
}

// Store the tile: output row m0 + r (r < rows_valid) of y with leading dimension ldy.
__device__ __forceinline__ void store_tile(const v16f (&acc)[2][4], float* __restrict__ y, int64_t ldy, int64_t m0,
                                           int64_t rows_valid, int64_t n0, int64_t O) {
  const int tid = threadIdx.x;
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
        const int rr = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (rr < rows_valid && o < O) y[(m0 + rr) * ldy + o] = acc[i][j][r];
      }
    }
}

// Plain two-path GEMM. Tiles are assigned so that each XCD (workgroups are
// dispatched round-robin over 8 XCDs) receives a contiguous range of tiles;
// inside a range consecutive tiles share a weight column tile.
// LDS of the main loops: the ring path uses four stage objects, the general
// path the first two as one contiguous double buffer.
#define SHARQ_GEMM_LDS                                                                    \
  __shared__ __attribute__((aligned(16))) uint8_t lds_s0[kStage];                         \
  __shared__ __attribute__((aligned(16))) uint8_t lds_s1[kStage];                         \
  __shared__ __attribute__((aligned(16))) uint8_t lds_s2[kRingPath ? kStage : 16];        \
  __shared__ __attribute__((aligned(16))) uint8_t lds_s3[kRingPath ? kStage : 16];

template <bool kRingPath>
__global__ __launch_bounds__(kThreads) void linear_kernel(Operands op, int64_t T, float* __restrict__ y,
                                                          int64_t ldy, int tiles_m, int tiles_total) {
  SHARQ_GEMM_LDS
  int tile = blockIdx.x;
  if ((tiles_total & 7) == 0) {
    const int per_xcd = tiles_total >> 3;
    tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  }
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  TileRows tr;
  tr.m0 = (int64_t)tm * kBM;
  tr.rows_valid = T - tr.m0 < kBM ? T - tr.m0 : kBM;
  tr.gather = nullptr;
  const int64_t n0 = (int64_t)tn * kBN;
  v16f acc[2][4];
  zero_acc(acc);
  if constexpr (kRingPath)
    mainloop_ring(op, tr, n0, RingStages{{lds_s0, lds_s1, lds_s2, lds_s3}}, acc);
  else
    mainloop_regs(op, tr, n0, lds_s0, lds_s1, acc);
  store_tile(acc, y, ldy, tr.m0, tr.rows_valid, n0, op.O);
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
template <bool kRingPath>
__global__ __launch_bounds__(kThreads) void linear_grouped_kernel(
    Operands op, const int32_t* __restrict__ a_rows, const int32_t* __restrict__ seg, int E,
    const uint8_t* __restrict__ w_codes_all, const uint8_t* __restrict__ w_scales_all, float* __restrict__ y) {
  SHARQ_GEMM_LDS
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
  TileRows tr;
  tr.m0 = seg[e] + (int64_t)s_info[1] * kBM;
  const int64_t hi = seg[e + 1];
  tr.rows_valid = hi - tr.m0 < kBM ? hi - tr.m0 : kBM;
  tr.gather = a_rows;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  op.w_codes = w_codes_all + (int64_t)e * op.O * kRowBytes * op.nsteps;  // [E][G][O][64]
  op.w_scales = w_scales_all + (int64_t)e * op.O * 4 * op.nsteps;          // [E][G][O][4]
  v16f acc[2][4];
  zero_acc(acc);
  if constexpr (kRingPath)
    mainloop_ring(op, tr, n0, RingStages{{lds_s0, lds_s1, lds_s2, lds_s3}}, acc);
  else
    mainloop_regs(op, tr, n0, lds_s0, lds_s1, acc);
  store_tile(acc, y, op.O, tr.m0, tr.rows_valid, n0, op.O);
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

}  // namespace

hipError_t launch_linear(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  const Operands op = make_operands(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K);
  const int tiles_m = (int)((T + kBM - 1) / kBM);
  const int tiles_n = (int)((O + kBN - 1) / kBN);
  const int total = tiles_m * tiles_n;
  if (ring_path_ok(T, O, K))
    hipLaunchKernelGGL(linear_kernel<true>, dim3(total), dim3(kThreads), 0, stream, op, T, y, ldy, tiles_m, total);
  else
    hipLaunchKernelGGL(linear_kernel<false>, dim3(total), dim3(kThreads), 0, stream, op, T, y, ldy, tiles_m, total);
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
  const int64_t tiles_m_bound = (P + kBM - 1) / kBM + E;
  const int tiles_n = (int)((O + kBN - 1) / kBN);
  const dim3 grid(tiles_n, (unsigned)tiles_m_bound);
  if (ring_path_ok(a_rows_total, O, K))
    hipLaunchKernelGGL(linear_grouped_kernel<true>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets, E,
                       w_codes, w_scales, y);
  else
    hipLaunchKernelGGL(linear_grouped_kernel<false>, grid, dim3(kThreads), 0, stream, op, a_rows, seg_offsets, E,
                       w_codes, w_scales, y);
  return hipGetLastError();
}

}  // namespace sharq

