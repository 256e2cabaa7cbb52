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

template <int N, int M>
__global__ __launch_bounds__(256) void compress_backbone_kernel(const uint8_t* __restrict__ bb_codes,
                                                                const uint8_t* __restrict__ mask, int64_t T,
                                                                int64_t K, uint32_t stages,
                                                                uint8_t* __restrict__ codes_out,
                                                                uint8_t* __restrict__ meta_out) {
  const Segment sg = segment_of_lane(stages, T);
  if (!sg.row_ok || (int64_t)sg.j * 64 >= K) return;
  const int64_t t = sg.t;
  // dense codes of blocks 2j and 2j + 1: 32 contiguous bytes in the stage-major layout
  const uint4 c0 = *reinterpret_cast<const uint4*>(bb_codes + code_offset(t, 2 * sg.j, T));
  const uint4 c1 = *reinterpret_cast<const uint4*>(bb_codes + code_offset(t, 2 * sg.j + 1, T));
  const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const uint2 mw = *reinterpret_cast<const uint2*>(mask + t * (K / 8) + 8 * (int64_t)sg.j);
  const uint64_t keep = (uint64_t)mw.x | ((uint64_t)mw.y << 32);
  // kept codes in index order, 8 nibbles per output word
  uint32_t out[4] = {0, 0, 0, 0};
  uint32_t k = 0;
#pragma unroll
  for (int p = 0; p < 64; ++p) {
    const uint32_t nib = (cw[p >> 3] >> (4 * (p & 7))) & 0xFu;
    if ((keep >> p) & 1u) {
      const uint32_t kk = k < 32 ? k : 31;  // a well-formed mask keeps exactly 32
      out[kk >> 3] |= nib << (4 * (kk & 7));
      ++k;
    }
  }
  *reinterpret_cast<uint4*>(codes_out + t * (K / 4) + 16 * (int64_t)sg.j) = make_uint4(out[0], out[1], out[2], out[3]);
  // one field per group: the colex rank of its kept positions
  constexpr int kB = field_bits<M>();
  uint64_t fields = 0;
#pragma unroll
  for (int g = 0; g < 64 / M; ++g) {
    uint32_t rank = 0, i = 0;
#pragma unroll
    for (int p = 0; p < M; ++p) {
      if ((keep >> (g * M + p)) & 1u) {
        ++i;
        rank += kBinom.c[p][i < 8 ? i : 8];
      }
    }
    fields |= (uint64_t)(rank & ((1u << kB) - 1)) << (g * kB);
  }
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
  // kept positions of each group: the largest p with C(p, i) <= rank is c_i, then i - 1 below it
  constexpr int kB = field_bits<M>();
  uint64_t keep = 0;
#pragma unroll
  for (int g = 0; g < 64 / M; ++g) {
    uint32_t r = (uint32_t)(fields >> (g * kB)) & ((1u << kB) - 1);
    int i = N;
#pragma unroll
    for (int p = M - 1; p >= 0; --p) {
      if (i > 0 && kBinom.c[p][i] <= r) {
        r -= kBinom.c[p][i];
        keep |= 1ull << (g * M + p);
        --i;
      }
    }
  }
  const uint4 cin = *reinterpret_cast<const uint4*>(codes_in + t * (K / 4) + 16 * (int64_t)sg.j);
  const uint32_t kw[4] = {cin.x, cin.y, cin.z, cin.w};
  uint32_t dense[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t k = 0;
#pragma unroll
  for (int p = 0; p < 64; ++p) {
    if ((keep >> p) & 1u) {
      const uint32_t kk = k < 32 ? k : 31;
      dense[p >> 3] |= ((kw[kk >> 3] >> (4 * (kk & 7))) & 0xFu) << (4 * (p & 7));
      ++k;
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
