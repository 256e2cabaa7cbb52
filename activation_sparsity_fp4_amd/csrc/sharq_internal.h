// Launchers behind the C ABI. Arguments reaching these have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

// rms_scale == nullptr: no RMSNorm; otherwise r per row is written there and
// absorbed (rms_eps > 0).
hipError_t launch_prepare(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma,
                          float rms_eps, float* rms_scale, int n, int m, uint8_t* bb_codes, uint8_t* bb_scales,
                          uint8_t* res_codes, uint8_t* res_scales, uint8_t* mask, hipStream_t stream);

hipError_t launch_quantize(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

hipError_t launch_linear(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream);

int64_t linear_workspace_bytes(int64_t T, int64_t O, int64_t K);
int64_t linear_silu_prepare_workspace_bytes(int64_t T, int64_t I, int64_t K);

hipError_t launch_linear_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                            const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales, int64_t T,
                            int64_t O, int64_t K, float* y, int64_t ldy, void* workspace, int64_t workspace_bytes,
                            hipStream_t stream);

// The scratch-free split-K GEMM (scratchfree.hip): whether the split plan's
// partials fit its static array, and the launch.
bool linear_scratchfree_fits(int64_t T, int64_t O, int64_t K);
hipError_t launch_linear_scratchfree(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                     const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                     int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream);

hipError_t launch_linear_grouped(const uint8_t* bb_codes, const uint8_t* bb_scales,
                                 const uint8_t* res_codes, const uint8_t* res_scales,
                                 const int32_t* a_rows, const int32_t* seg_offsets, int32_t E,
                                 const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t O,
                                 int64_t K, float* y, int64_t a_rows_total, hipStream_t stream);

hipError_t launch_linear_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                      const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                      int64_t T, int64_t I, int64_t K, int n, int m, uint16_t* h,
                                      uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                      uint8_t* h_res_scales, uint8_t* h_mask, hipStream_t stream);

hipError_t launch_linear_silu_prepare_ws(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                         const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                         int64_t T, int64_t I, int64_t K, int n, int m, uint16_t* h,
                                         uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                         uint8_t* h_res_scales, uint8_t* h_mask, void* workspace,
                                         int64_t workspace_bytes, hipStream_t stream);

hipError_t launch_linear_grouped_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales,
                                              const uint8_t* res_codes, const uint8_t* res_scales,
                                              const int32_t* a_rows, const int32_t* seg_offsets, int32_t E,
                                              const uint8_t* w_codes, const uint8_t* w_scales, int64_t P, int64_t I,
                                              int64_t K, int64_t a_rows_total, int n, int m, uint16_t* h,
                                              uint8_t* h_bb_codes, uint8_t* h_bb_scales, uint8_t* h_res_codes,
                                              uint8_t* h_res_scales, uint8_t* h_mask, hipStream_t stream);

int64_t backbone_meta_row_bytes(int64_t K, int m);

hipError_t launch_compress_backbone(const uint8_t* bb_codes, const uint8_t* mask, int64_t T, int64_t K, int n, int m,
                                    uint8_t* codes, uint8_t* meta, hipStream_t stream);

hipError_t launch_expand_backbone(const uint8_t* codes, const uint8_t* meta, int64_t T, int64_t K, int n, int m,
                                  uint8_t* bb_codes, uint8_t* mask, hipStream_t stream);

hipError_t launch_moe_combine(const float* y, int64_t P, int64_t H, const int32_t* pair_index, const float* weights,
                              int64_t T, int k, float* out, uint16_t* out_bf16, hipStream_t stream);

hipError_t launch_prepare_nvfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx, const uint16_t* gamma, int n,
                                int m, float s_t, uint8_t* bb_codes, uint8_t* bb_scales, uint8_t* res_codes,
                                uint8_t* res_scales, uint8_t* mask, hipStream_t stream);

hipError_t launch_quantize_nvfp4(const uint16_t* w, int64_t O, int64_t K, int64_t ldw, float s_t, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

hipError_t launch_linear_nvfp4(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                               const uint8_t* res_scales, float s_a, const uint8_t* w_codes, const uint8_t* w_scales,
                               float s_w, int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                               hipStream_t stream);

hipError_t launch_pack(const uint8_t* codes_rm, const uint8_t* scales_rm, int64_t R, int64_t K, int block,
                       uint8_t* codes, uint8_t* scales, hipStream_t stream);

hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t K, int block,
                         uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t stream);

hipError_t launch_silu_mul(const float* gu, int64_t T, int64_t I, uint16_t* h, hipStream_t stream);

}  // namespace sharq
