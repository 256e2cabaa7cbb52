// Compressed sparse backbone for gfx950: the "sparse input compression" the
// SharQ page names in its Abstract (no format is given there). With N of every
// M positions kept, the backbone's dense-masked codes carry M - N zero codes
// per group; the compressed form keeps only the N kept codes of each group in
// index order, plus one field per group naming which positions were kept. The
// field is the rank of the kept set in the combinatorial number system
// (colexicographic order): for kept positions c_1 < ... < c_N inside the
// group, rank = C(c_1, 1) + ... + C(c_N, N), which takes ceil(log2 C(M, N))
// bits: 3 bits per 4 entries for 2:4 and 14 bits per 16 for 8:16, the 0.75
// and 0.875 bits per element the 8:16 page (abstract) gives for storing an
// N:M mask. A row's fields form a bit stream, group g at bits [g b, g b + b),
// least significant bit first. Block scales are unchanged.
//
// gfx950 has no structured-sparse FP4 MFMA, so the GEMM runs on the dense
// form; the compressed form is for storing or moving a prepared activation
// (for example the FP4 activations exchanged between GPUs of a sharded
// linear layer): backbone codes shrink from 0.5 to 0.25 bytes per element
// and the mask from 0.125 to 0.094 (2:4) or 0.109 (8:16).
//
// Work decomposition: one lane owns a 64-entry segment (two MX blocks) of one
// row: 32 kept codes (16 bytes) and 16 (2:4) or 4 (8:16) fields, i.e. 6 or 7
// whole bytes of the row's bit stream, so no two lanes share a byte. A wave
// covers 32 rows of one 128-entry stage, so its dense code accesses are one
// contiguous 2 KB run in the stage-major layout.

#include "sharq_device.h"
#include "sharq_internal.h"

namespace sharq {

namespace {

// C(p, i) for p < 16, i <= 8 by Pascal's rule, built at compile time.
struct Binomials {
  uint32_t c[17][9];
  constexpr Binomials() : c{} {
    for (int p = 0; p <= 16; ++p) {
      c[p][0] = 1;
      for (int i = 1; i <= 8; ++i) c[p][i] = p == 0 ? 0 : c[p - 1][i - 1] + c[p - 1][i];
    }
  }
};
__constant__ Binomials kBinom = Binomials();

template <int M>
constexpr int field_bits() {
  return M == 4 ? 3 : 14;  // ceil(log2 C(4, 2)) and ceil(log2 C(16, 8))
}
template <int M>
constexpr int segment_meta_bytes() {
  return 64 / M * field_bits<M>() / 8;  // 6 (2:4) or 7 (8:16)
}

struct Segment {
  int64_t t;
  uint32_t j;      // 64-entry segment of the row
  bool row_ok;
};

// Lane -> (row, segment): a wave owns 32 rows of one 128-entry stage
// (2 segments), lane l row 32 * band + l / 2, segment 2 * stage + l % 2.
__device__ __forceinline__ Segment segment_of_lane(uint32_t stages, int64_t rows) {
  const uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t wave = gid >> 6;
  const uint32_t lane = gid & 63;
  const uint64_t band = wave / stages;
  const uint32_t g = (uint32_t)(wave - band * stages);
  Segment s;
  s.t = (int64_t)(band * 32 + (lane >> 1));
  s.j = 2 * g + (lane & 1);
  s.row_ok = s.t < rows;
  return s;
}

// C(c, i) for 0 <= c < 16, 1 <= i <= N (c and i per lane): in closed form
// for 2:4 (i <= 2), from the workgroup's LDS copy of the table otherwise.
template <int M>
__device__ __forceinline__ uint32_t binom(const uint32_t* lds_table, uint32_t c, uint32_t i) {
  if constexpr (M == 4) {
    return i == 1 ? c : c * (c - 1) / 2;
  } else {
    return lds_table[c * 9 + i];
  }
}

// Every thread of the workgroup takes part (before any early return).
template <int M>
__device__ __forceinline__ void load_binomials(uint32_t* lds_table) {
  if constexpr (M != 4) {
    for (uint32_t q = threadIdx.x; q < 17 * 9; q += blockDim.x) lds_table[q] = (&kBinom.c[0][0])[q];
    __syncthreads();
  }
}

template <int N, int M>
__global__ __launch_bounds__(256) void compress_backbone_kernel(const uint8_t* __restrict__ bb_codes,
                                                                const uint8_t* __restrict__ mask, int64_t T,
                                                                int64_t K, uint32_t stages,
                                                                uint8_t* __restrict__ codes_out,
                                                                uint8_t* __restrict__ meta_out) {
  __shared__ uint32_t table[17 * 9];
  load_binomials<M>(table);
  const Segment sg = segment_of_lane(stages, T);
  if (!sg.row_ok || (int64_t)sg.j * 64 >= K) return;
  const int64_t t = sg.t;
  // dense codes of blocks 2j and 2j + 1: 32 contiguous bytes in the stage-major layout
  const uint4 c0 = *reinterpret_cast<const uint4*>(bb_codes + code_offset(t, 2 * sg.j, T));
  const uint4 c1 = *reinterpret_cast<const uint4*>(bb_codes + code_offset(t, 2 * sg.j + 1, T));
  const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const uint2 mw = *reinterpret_cast<const uint2*>(mask + t * (K / 8) + 8 * (int64_t)sg.j);
  const uint64_t keep = (uint64_t)mw.x | ((uint64_t)mw.y << 32);
  // per group: the kept positions in increasing order (lowest set bit first)
  // give both the kept codes, in index order, and the rank C(c_1, 1) + ...
  constexpr int kB = field_bits<M>();
  constexpr int kGroups = 64 / M;
  uint32_t out[4] = {0, 0, 0, 0};
  uint64_t fields = 0;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    // the group's 4 M code bits, position 0 lowest
    uint64_t gc;
    if constexpr (M == 4) {
      gc = (cw[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
    } else {
      gc = (uint64_t)cw[2 * g] | ((uint64_t)cw[2 * g + 1] << 32);
    }
    uint32_t gm = (uint32_t)(keep >> (g * M)) & ((1u << M) - 1);
    uint32_t rank = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t c = gm ? (uint32_t)__builtin_ctz(gm) : 0;  // a well-formed group has N set bits
      gm &= gm - 1;
      const uint32_t nib = (uint32_t)(gc >> (4 * c)) & 0xFu;
      const int k = g * N + i;  // output nibble (compile-time)
      out[k >> 3] |= nib << (4 * (k & 7));
      rank += binom<M>(table, c, i + 1);
    }
    fields |= (uint64_t)(rank & ((1u << kB) - 1)) << (g * kB);
  }
  *reinterpret_cast<uint4*>(codes_out + t * (K / 4) + 16 * (int64_t)sg.j) = make_uint4(out[0], out[1], out[2], out[3]);
  uint8_t* dst = meta_out + t * (K / 64 * segment_meta_bytes<M>()) + (int64_t)sg.j * segment_meta_bytes<M>();
#pragma unroll
  for (int q = 0; q < segment_meta_bytes<M>(); ++q) dst[q] = (uint8_t)(fields >> (8 * q));
}

template <int N, int M>
__global__ __launch_bounds__(256) void expand_backbone_kernel(const uint8_t* __restrict__ codes_in,
                                                              const uint8_t* __restrict__ meta_in, int64_t T,
                                                              int64_t K, uint32_t stages,
                                                              uint8_t* __restrict__ bb_codes,
                                                              uint8_t* __restrict__ mask) {
  __shared__ uint32_t table[17 * 9];
  load_binomials<M>(table);
  const Segment sg = segment_of_lane(stages, T);
  if (!sg.row_ok) return;
  const int64_t t = sg.t;
  if ((int64_t)sg.j * 64 >= K) {
    // the unused blocks of a last, partial stage are zero
    *reinterpret_cast<uint4*>(bb_codes + code_offset(t, 2 * sg.j, T)) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(bb_codes + code_offset(t, 2 * sg.j + 1, T)) = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint8_t* src = meta_in + t * (K / 64 * segment_meta_bytes<M>()) + (int64_t)sg.j * segment_meta_bytes<M>();
  uint64_t fields = 0;
#pragma unroll
  for (int q = 0; q < segment_meta_bytes<M>(); ++q) fields |= (uint64_t)src[q] << (8 * q);
  const uint4 cin = *reinterpret_cast<const uint4*>(codes_in + t * (K / 4) + 16 * (int64_t)sg.j);
  const uint32_t kw[4] = {cin.x, cin.y, cin.z, cin.w};
  // per group, the kept positions from the rank: scanning p = M-1 .. 0, p is
  // the next (largest remaining) kept position c_i when C(p, i) <= the rank
  // left; the i-th kept code (in index order) goes to position c_i
  constexpr int kB = field_bits<M>();
  constexpr int kGroups = 64 / M;
  uint32_t dense[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint64_t keep = 0;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    uint32_t r = (uint32_t)(fields >> (g * kB)) & ((1u << kB) - 1);
    uint32_t i = N;
    uint32_t gm = 0;
#pragma unroll
    for (int p = M - 1; p >= 0; --p) {
      const uint32_t cb = binom<M>(table, (uint32_t)p, i > 0 ? i : 1);
      const bool take = i > 0 && cb <= r;
      r -= take ? cb : 0;
      gm |= take ? 1u << p : 0u;
      i -= take ? 1 : 0;
    }
    keep |= (uint64_t)gm << (g * M);
    uint64_t gd = 0;  // the group's dense code bits
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const uint32_t c = gm ? (uint32_t)__builtin_ctz(gm) : 0;
      gm &= gm - 1;
      const int k = g * N + q;  // compressed nibble (compile-time)
      gd |= (uint64_t)((kw[k >> 3] >> (4 * (k & 7))) & 0xFu) << (4 * c);
    }
    if constexpr (M == 4) {
      dense[g >> 1] |= (uint32_t)gd << (16 * (g & 1));
    } else {
      dense[2 * g] = (uint32_t)gd;
      dense[2 * g + 1] = (uint32_t)(gd >> 32);
    }
  }
  *reinterpret_cast<uint4*>(bb_codes + code_offset(t, 2 * sg.j, T)) = make_uint4(dense[0], dense[1], dense[2], dense[3]);
  *reinterpret_cast<uint4*>(bb_codes + code_offset(t, 2 * sg.j + 1, T)) =
      make_uint4(dense[4], dense[5], dense[6], dense[7]);
  if (mask)
    *reinterpret_cast<uint2*>(mask + t * (K / 8) + 8 * (int64_t)sg.j) =
        make_uint2((uint32_t)keep, (uint32_t)(keep >> 32));
}

dim3 segment_grid(int64_t T, uint32_t stages) {
  const uint64_t lanes = (uint64_t)((T + 31) / 32) * stages * 64;
  return dim3((unsigned)((lanes + 255) / 256));
}

}  // namespace

int64_t backbone_meta_row_bytes(int64_t K, int m) { return K / 64 * (m == 4 ? 6 : 7); }

hipError_t launch_compress_backbone(const uint8_t* bb_codes, const uint8_t* mask, int64_t T, int64_t K, int n, int m,
                                    uint8_t* codes, uint8_t* meta, hipStream_t stream) {
  const uint32_t stages = (uint32_t)((K + 127) / 128);
  if (n == 2 && m == 4)
    hipLaunchKernelGGL((compress_backbone_kernel<2, 4>), segment_grid(T, stages), dim3(256), 0, stream, bb_codes,
                       mask, T, K, stages, codes, meta);
  else
    hipLaunchKernelGGL((compress_backbone_kernel<8, 16>), segment_grid(T, stages), dim3(256), 0, stream, bb_codes,
                       mask, T, K, stages, codes, meta);
  return hipGetLastError();
}

hipError_t launch_expand_backbone(const uint8_t* codes, const uint8_t* meta, int64_t T, int64_t K, int n, int m,
                                  uint8_t* bb_codes, uint8_t* mask, hipStream_t stream) {
  const uint32_t stages = (uint32_t)((K + 127) / 128);
  if (n == 2 && m == 4)
    hipLaunchKernelGGL((expand_backbone_kernel<2, 4>), segment_grid(T, stages), dim3(256), 0, stream, codes, meta, T,
                       K, stages, bb_codes, mask);
  else
    hipLaunchKernelGGL((expand_backbone_kernel<8, 16>), segment_grid(T, stages), dim3(256), 0, stream, codes, meta,
                       T, K, stages, bb_codes, mask);
  return hipGetLastError();
}

}  // namespace sharq
