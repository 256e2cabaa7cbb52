// C ABI of the SharQ library: host-side argument validation (before any HIP
// call) and dispatch to the kernel launchers.

#include <math.h>

#include "../../include/sharq.h"
#include "sharq_internal.h"

namespace {

constexpr int kAbiVersion = 10;
// Workgroups of one grouped launch: a one-dimensional grid of 256-thread
// workgroups whose thread count must stay below 2^32.
constexpr int64_t kMaxGroupedTiles = (int64_t)1 << 24;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? SHARQ_OK : SHARQ_EHIP; }

// Shape checks shared by sharq_prepare and sharq_quantize_mxfp4.
int check_rows(int64_t T, int64_t K, int64_t ldx) {
  if (T < 0 || K <= 0 || K % 32 != 0 || ldx < K) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T * (K / 32) >= ((int64_t)1 << 31)) return SHARQ_EINVAL;  // 32-bit block index
  if (ldx % 8 != 0) return SHARQ_EALIGN;
  return SHARQ_OK;
}

}  // namespace

namespace {

// Argument checks shared by sharq_linear_silu_prepare and its split-K form.
int check_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                       const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T,
                       int64_t I, int64_t K, int n, int m, uint16_t* h, uint8_t* h_bb_codes, uint8_t* h_bb_scales,
                       uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  if (T < 0 || I <= 0 || K <= 0 || K % 32 != 0 || I % 32 != 0) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || I >= ((int64_t)1 << 30) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T * (I / 32) >= ((int64_t)1 << 31)) return SHARQ_EINVAL;  // 32-bit block index of the h blocks
  if (I % 128 != 0 || K % 128 != 0) return SHARQ_ENOTIMPL;     // whole 128-column h tiles, ring path only
  if (T * (K / 2) >= ((int64_t)1 << 31) || 2 * I * (K / 2) >= ((int64_t)1 << 31)) return SHARQ_ENOTIMPL;
  const bool prep = h_bb_codes || h_bb_scales || h_res_codes || h_res_scales;
  if (prep && !(h_bb_codes && h_bb_scales && h_res_codes && h_res_scales)) return SHARQ_EINVAL;
  if (!prep && h_mask) return SHARQ_EINVAL;
  if (!prep && !h) return SHARQ_EINVAL;  // nothing to write
  if (T == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !w_codes || !w_scales) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || (h && !aligned16(h)) ||
      (prep && (!aligned16(h_bb_codes) || !aligned16(h_bb_scales) || !aligned16(h_res_codes) ||
                !aligned16(h_res_scales))) ||
      (h_mask && !aligned16(h_mask)))
    return SHARQ_EALIGN;
  return SHARQ_OK;
}

}  // namespace

namespace {

// Shape checks of the compressed-backbone entry points.
int check_compact(int64_t T, int64_t K, int n, int m) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  if (T < 0 || K <= 0 || K % 32 != 0) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31) || T * (K / 32) >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (K % 64 != 0) return SHARQ_ENOTIMPL;
  return SHARQ_OK;
}

}  // namespace

extern "C" {

const char* sharq_status_string(int status) {
  switch (status) {
    case SHARQ_OK: return "ok";
    case SHARQ_EINVAL: return "invalid argument (shape, stride or NULL pointer)";
    case SHARQ_EALIGN: return "misaligned pointer or leading dimension";
    case SHARQ_EUNSUPPORTED: return "unsupported N:M pattern (supported: 2:4, 8:16)";
    case SHARQ_EHIP: return "HIP launch failed";
    case SHARQ_ENOTIMPL: return "not implemented";
    case SHARQ_ESCRATCH: return "the call needs more scratch memory than the static maximum";
    default: return "unknown status";
  }
}

int sharq_abi_version(void) { return kAbiVersion; }

int sharq_prepare(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma, int n, int m,
                  uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes, uint8_t* res_scales, uint8_t* mask,
                  hipStream_t stream) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  const int rc = check_rows(T, K, ldx);
  if (rc != SHARQ_OK) return rc;
  if (K % m != 0) return SHARQ_EINVAL;
  if (T == 0) return SHARQ_OK;
  if (!x || !bb_codes || !bb_scales || !res_codes || !res_scales) return SHARQ_EINVAL;
  if (!aligned16(x) || (gamma && !aligned16(gamma)) || !aligned16(bb_codes) || !aligned16(bb_scales) ||
      !aligned16(res_codes) || !aligned16(res_scales) || (mask && !aligned16(mask)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_prepare(x, T, K, ldx, gamma, 0.0f, nullptr, n, m, bb_codes, bb_scales, res_codes,
                                          res_scales, mask, stream));
}

int sharq_prepare_rms(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma, float eps,
                      int n, int m, float* rms_scale, uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes,
                      uint8_t* res_scales, uint8_t* mask, hipStream_t stream) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  const int rc = check_rows(T, K, ldx);
  if (rc != SHARQ_OK) return rc;
  if (K % m != 0 || !(eps > 0.0f) || !(eps < INFINITY)) return SHARQ_EINVAL;
  if (K / 32 > 4096) return SHARQ_ENOTIMPL;  // the row-sum tree holds at most 4096 blocks
  if (T == 0) return SHARQ_OK;
  if (!x || !rms_scale || !bb_codes || !bb_scales || !res_codes || !res_scales) return SHARQ_EINVAL;
  if (!aligned16(x) || (gamma && !aligned16(gamma)) || !aligned16(rms_scale) || !aligned16(bb_codes) ||
      !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) || (mask && !aligned16(mask)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_prepare(x, T, K, ldx, gamma, eps, rms_scale, n, m, bb_codes, bb_scales,
                                          res_codes, res_scales, mask, stream));
}

int sharq_quantize_mxfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, uint8_t* codes, uint8_t* scales,
                         hipStream_t stream) {
  const int rc = check_rows(T, K, ldx);
  if (rc != SHARQ_OK) return rc;
  if (T == 0) return SHARQ_OK;
  if (!x || !codes || !scales) return SHARQ_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_quantize(x, T, K, ldx, codes, scales, stream));
}

int sharq_prepare_nvfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma, int n, int m,
                        float tensor_scale, uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes,
                        uint8_t* res_scales, uint8_t* mask, hipStream_t stream) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  const int rc = check_rows(T, K, ldx);
  if (rc != SHARQ_OK) return rc;
  if (K % m != 0 || !(tensor_scale > 0.0f) || !(tensor_scale < INFINITY)) return SHARQ_EINVAL;
  if (T == 0) return SHARQ_OK;
  if (!x || !bb_codes || !bb_scales || !res_codes || !res_scales) return SHARQ_EINVAL;
  if (!aligned16(x) || (gamma && !aligned16(gamma)) || !aligned16(bb_codes) || !aligned16(bb_scales) ||
      !aligned16(res_codes) || !aligned16(res_scales) || (mask && !aligned16(mask)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_prepare_nvfp4(x, T, K, ldx, gamma, n, m, tensor_scale, bb_codes, bb_scales,
                                                res_codes, res_scales, mask, stream));
}

int sharq_quantize_nvfp4(const uint16_t* w, int64_t O, int64_t K, int64_t ldw, float tensor_scale, uint8_t* codes,
                         uint8_t* scales, hipStream_t stream) {
  const int rc = check_rows(O, K, ldw);
  if (rc != SHARQ_OK) return rc;
  if (!(tensor_scale > 0.0f) || !(tensor_scale < INFINITY)) return SHARQ_EINVAL;
  if (O == 0) return SHARQ_OK;
  if (!w || !codes || !scales) return SHARQ_EINVAL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_quantize_nvfp4(w, O, K, ldw, tensor_scale, codes, scales, stream));
}

int sharq_linear_nvfp4(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                       const uint8_t* res_scales, float a_tensor_scale, const uint8_t* w_codes,
                       const uint8_t* w_scales, float w_tensor_scale, int64_t T, int64_t O, int64_t K, float* y,
                       int64_t ldy, hipStream_t stream) {
  if (T < 0 || O < 0 || K <= 0 || K % 32 != 0 || ldy < O) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (!(a_tensor_scale > 0.0f) || !(a_tensor_scale < INFINITY) || !(w_tensor_scale > 0.0f) ||
      !(w_tensor_scale < INFINITY))
    return SHARQ_EINVAL;
  if (((T + 127) / 128) * ((O + 255) / 256) > ((int64_t)1 << 24)) return SHARQ_EINVAL;  // one-dimensional grid
  if (T == 0 || O == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !w_codes || !w_scales || !y) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_linear_nvfp4(bb_codes, bb_scales, res_codes, res_scales, a_tensor_scale, w_codes,
                                               w_scales, w_tensor_scale, T, O, K, y, ldy, stream));
}

int sharq_linear(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                 const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T, int64_t O,
                 int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  if (T < 0 || O < 0 || K <= 0 || K % 32 != 0 || ldy < O) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T == 0 || O == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !w_codes || !w_scales || !y) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y))
    return SHARQ_EALIGN;
  return hip_status(
      sharq::launch_linear(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K, y, ldy, stream));
}

int64_t sharq_linear_workspace_bytes(int64_t T, int64_t O, int64_t K) {
  if (T < 0 || O < 0 || K <= 0 || K % 32 != 0) return 0;
  if (T >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return 0;
  return sharq::linear_workspace_bytes(T, O, K);
}

int sharq_linear_scratchfree(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                             const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T,
                             int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  if (T < 0 || O < 0 || K <= 0 || K % 32 != 0 || ldy < O) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T == 0 || O == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !w_codes || !w_scales || !y) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y))
    return SHARQ_EALIGN;
  if (!sharq::linear_scratchfree_fits(T, O, K)) return SHARQ_ESCRATCH;
  return hip_status(sharq::launch_linear_scratchfree(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales,
                                                     T, O, K, y, ldy, stream));
}

int sharq_linear_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                    const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T, int64_t O,
                    int64_t K, float* y, int64_t ldy, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || O < 0 || K <= 0 || K % 32 != 0 || ldy < O || workspace_bytes < 0) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T == 0 || O == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !w_codes || !w_scales || !y) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y) || (workspace && !aligned16(workspace)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_linear_ws(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K,
                                            y, ldy, workspace, workspace_bytes, stream));
}

int sharq_linear_grouped(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                         const uint8_t* res_scales, int64_t T_src, const int32_t* a_rows, const int32_t* seg_offsets,
                         int32_t E, const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t O, int64_t K,
                         float* y, hipStream_t stream) {
  if (E < 1 || P < 0 || O < 0 || K <= 0 || K % 32 != 0 || T_src < 0) return SHARQ_EINVAL;
  if (!a_rows && T_src < P) return SHARQ_EINVAL;
  if (T_src >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (P >= ((int64_t)1 << 31) || O >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31) ||
      ((P + 127) / 128 + E) * ((O + 255) / 256) > kMaxGroupedTiles)
    return SHARQ_EINVAL;
  if (P == 0 || O == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !seg_offsets || !w_codes || !w_scales || !y)
    return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(y) || !aligned16(seg_offsets) ||
      (a_rows && !aligned16(a_rows)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_linear_grouped(bb_codes, bb_scales, res_codes, res_scales, a_rows, seg_offsets,
                                                 E, w_codes, w_scales, P, O, K, y, T_src, stream));
}


int sharq_linear_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                              const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T,
                              int64_t I, int64_t K, int n, int m, uint16_t* h, uint8_t* h_bb_codes,
                              uint8_t* h_bb_scales, uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask,
                              hipStream_t stream) {
  const int rc = check_silu_prepare(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, I, K, n, m, h,
                                    h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask);
  if (rc != SHARQ_OK || T == 0) return rc;
  return hip_status(sharq::launch_linear_silu_prepare(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales,
                                                      T, I, K, n, m, h, h_bb_codes, h_bb_scales, h_res_codes,
                                                      h_res_scales, h_mask, stream));
}

int64_t sharq_linear_silu_prepare_workspace_bytes(int64_t T, int64_t I, int64_t K) {
  if (T <= 0 || I <= 0 || K <= 0 || I % 128 != 0 || K % 128 != 0) return 0;
  if (T >= ((int64_t)1 << 31) || I >= ((int64_t)1 << 30) || K >= ((int64_t)1 << 31)) return 0;
  return sharq::linear_silu_prepare_workspace_bytes(T, I, K);
}

int sharq_linear_silu_prepare_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                 const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                 int64_t T, int64_t I, int64_t K, int n, int m, uint16_t* h, uint8_t* h_bb_codes,
                                 uint8_t* h_bb_scales, uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask,
                                 void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  const int rc = check_silu_prepare(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, I, K, n, m, h,
                                    h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask);
  if (rc != SHARQ_OK || T == 0) return rc;
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return SHARQ_EINVAL;
  if (workspace && !aligned16(workspace)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_linear_silu_prepare_ws(bb_codes, bb_scales, res_codes, res_scales, w_codes,
                                                         w_scales, T, I, K, n, m, h, h_bb_codes, h_bb_scales,
                                                         h_res_codes, h_res_scales, h_mask, workspace,
                                                         workspace_bytes, stream));
}

int sharq_linear_grouped_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                      const uint8_t* res_scales, int64_t T_src, const int32_t* a_rows,
                                      const int32_t* seg_offsets, int32_t E, const uint8_t* w_codes,
                                      const uint8_t* w_scales, int64_t P, int64_t I, int64_t K, int n, int m,
                                      uint16_t* h, uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                      uint8_t* h_res_scales, uint8_t* h_mask, hipStream_t stream) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  if (E < 1 || P < 0 || I <= 0 || K <= 0 || K % 32 != 0 || I % 32 != 0 || T_src < 0) return SHARQ_EINVAL;
  if (!a_rows && T_src < P) return SHARQ_EINVAL;
  if (T_src >= ((int64_t)1 << 31) || P >= ((int64_t)1 << 31) || I >= ((int64_t)1 << 30) ||
      K >= ((int64_t)1 << 31) || ((P + 127) / 128 + E) * (I / 128) > kMaxGroupedTiles)
    return SHARQ_EINVAL;
  if (P * (I / 32) >= ((int64_t)1 << 31)) return SHARQ_EINVAL;  // 32-bit block index of the h blocks
  if (I % 128 != 0 || K % 128 != 0) return SHARQ_ENOTIMPL;     // whole 128-column h tiles, ring path only
  if (T_src * (K / 2) >= ((int64_t)1 << 31) || 2 * I * (K / 2) >= ((int64_t)1 << 31)) return SHARQ_ENOTIMPL;
  const bool prep = h_bb_codes || h_bb_scales || h_res_codes || h_res_scales;
  if (prep && !(h_bb_codes && h_bb_scales && h_res_codes && h_res_scales)) return SHARQ_EINVAL;
  if (!prep && h_mask) return SHARQ_EINVAL;
  if (!prep && !h) return SHARQ_EINVAL;
  if (P == 0) return SHARQ_OK;
  if (!bb_codes || !bb_scales || !res_codes || !res_scales || !seg_offsets || !w_codes || !w_scales)
    return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(bb_scales) || !aligned16(res_codes) || !aligned16(res_scales) ||
      !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(seg_offsets) || (a_rows && !aligned16(a_rows)) ||
      (h && !aligned16(h)) ||
      (prep && (!aligned16(h_bb_codes) || !aligned16(h_bb_scales) || !aligned16(h_res_codes) ||
                !aligned16(h_res_scales))) ||
      (h_mask && !aligned16(h_mask)))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_linear_grouped_silu_prepare(
      bb_codes, bb_scales, res_codes, res_scales, a_rows, seg_offsets, E, w_codes, w_scales, P, I, K, T_src, n, m, h,
      h_bb_codes, h_bb_scales, h_res_codes, h_res_scales, h_mask, stream));
}

int64_t sharq_backbone_meta_row_bytes(int64_t K, int n, int m) {
  if (!((n == 2 && m == 4) || (n == 8 && m == 16))) return SHARQ_EUNSUPPORTED;
  if (K <= 0 || K % 32 != 0) return SHARQ_EINVAL;
  if (K % 64 != 0) return SHARQ_ENOTIMPL;
  return sharq::backbone_meta_row_bytes(K, m);
}

int sharq_compress_backbone(const uint8_t* bb_codes, const uint8_t* mask, int64_t T, int64_t K, int n, int m,
                            uint8_t* codes, uint8_t* meta, hipStream_t stream) {
  const int rc = check_compact(T, K, n, m);
  if (rc != SHARQ_OK || T == 0) return rc;
  if (!bb_codes || !mask || !codes || !meta) return SHARQ_EINVAL;
  if (!aligned16(bb_codes) || !aligned16(mask) || !aligned16(codes)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_compress_backbone(bb_codes, mask, T, K, n, m, codes, meta, stream));
}

int sharq_expand_backbone(const uint8_t* codes, const uint8_t* meta, int64_t T, int64_t K, int n, int m,
                          uint8_t* bb_codes, uint8_t* mask, hipStream_t stream) {
  const int rc = check_compact(T, K, n, m);
  if (rc != SHARQ_OK || T == 0) return rc;
  if (!codes || !meta || !bb_codes) return SHARQ_EINVAL;
  if (!aligned16(codes) || !aligned16(bb_codes) || (mask && !aligned16(mask))) return SHARQ_EALIGN;
  return hip_status(sharq::launch_expand_backbone(codes, meta, T, K, n, m, bb_codes, mask, stream));
}

int sharq_moe_combine(const float* y, int64_t P, int64_t H, const int32_t* pair_index, const float* weights,
                      int64_t T, int32_t k, float* out, uint16_t* out_bf16, hipStream_t stream) {
  if (P < 0 || H <= 0 || H % 4 != 0 || T < 0 || k < 1 || k > 64) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || T * (H / 4) >= ((int64_t)1 << 32) - 256) return SHARQ_EINVAL;  // 32-bit lane index
  if (!out && !out_bf16) return SHARQ_EINVAL;  // nothing to write
  if (T == 0) return SHARQ_OK;
  if (!pair_index || !weights || (P > 0 && !y)) return SHARQ_EINVAL;
  if ((y && !aligned16(y)) || (out && !aligned16(out)) || (out_bf16 && ((uintptr_t)out_bf16 & 7u)) ||
      ((uintptr_t)pair_index & 3u) || ((uintptr_t)weights & 3u))
    return SHARQ_EALIGN;
  return hip_status(sharq::launch_moe_combine(y, P, H, pair_index, weights, T, k, out, out_bf16, stream));
}

namespace {

// Shape checks of the layout conversions.
int check_pack(int64_t R, int64_t K, int block) {
  if (block != 32 && block != 16) return SHARQ_EINVAL;
  if (R < 0 || K <= 0 || K % 32 != 0) return SHARQ_EINVAL;
  if (R >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if ((K + 127) / 128 * R * 64 >= ((int64_t)1 << 31)) return SHARQ_EINVAL;  // stage-major codes bytes
  return SHARQ_OK;
}

}  // namespace

int sharq_pack_stage_major(const uint8_t* codes_rm, const uint8_t* scales_rm, int64_t R, int64_t K, int block,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int rc = check_pack(R, K, block);
  if (rc != SHARQ_OK) return rc;
  if (R == 0) return SHARQ_OK;
  if (!codes_rm || !scales_rm || !codes || !scales) return SHARQ_EINVAL;
  if (!aligned16(codes_rm) || !aligned16(codes)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_pack(codes_rm, scales_rm, R, K, block, codes, scales, stream));
}

int sharq_unpack_stage_major(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t K, int block,
                             uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t stream) {
  const int rc = check_pack(R, K, block);
  if (rc != SHARQ_OK) return rc;
  if (R == 0) return SHARQ_OK;
  if (!codes_rm || !scales_rm || !codes || !scales) return SHARQ_EINVAL;
  if (!aligned16(codes_rm) || !aligned16(codes)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_unpack(codes, scales, R, K, block, codes_rm, scales_rm, stream));
}

int sharq_silu_mul(const float* gu, int64_t T, int64_t I, uint16_t* h, hipStream_t stream) {
  if (T < 0 || I <= 0 || I % 8 != 0) return SHARQ_EINVAL;
  if (T >= ((int64_t)1 << 31) || I >= ((int64_t)1 << 31)) return SHARQ_EINVAL;
  if (T * (I / 8) >= ((int64_t)1 << 32) - 256) return SHARQ_EINVAL;  // 32-bit lane index
  if (T == 0) return SHARQ_OK;
  if (!gu || !h) return SHARQ_EINVAL;
  if (!aligned16(gu) || !aligned16(h)) return SHARQ_EALIGN;
  return hip_status(sharq::launch_silu_mul(gu, T, I, h, stream));
}

}  // extern "C"
