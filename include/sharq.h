/*
 * sharq.h -- C ABI of the SharQ linear hot path on AMD MI355X (gfx950).
 *
 * The method (page "SharQ: Bridging Activation Sparsity and FP4 Quantization
 * for LLM Inference", Abstract and Section 1): for each activation row an
 * online N:M mask keeps the N largest |x| of every M consecutive entries along
 * K; that outlier-dominated sparse backbone is quantised to block-scaled FP4;
 * a dense residual is taken against the *quantised* backbone and quantised to
 * FP4 with its own scales; a sparse FP4 GEMM on the backbone and a dense FP4
 * GEMM on the residual share one FP4 weight and accumulate into one output.
 *
 * FP4 format (MXFP4, the OCP MX format named in Section 2.3 of that page):
 * E2M1 codes {0, .5, 1, 1.5, 2, 3, 4, 6} with bit 3 the sign, two codes per
 * byte with the even K index in the low nibble; one E8M0 scale byte
 * (exponent + 127) per 32 consecutive K entries; exponent
 * floor(log2(block amax)) - 2, clamped to [-127, 127], -127 for an all-zero
 * block; codes round to nearest with ties to the even code and saturate at 6.
 *
 * Layout ("stage-major"): a tensor of R rows and K entries per row is cut
 * into G = ceil(K / 128) stages of 128 K entries (4 blocks of 32), stored one
 * stage after the other:
 *   codes  u8 [G][R][64]: the 16 code bytes of block b (K entries
 *          [32 b, 32 b + 32)) of row r sit at [b / 4][r][16 (b % 4) .. +16),
 *          two codes per byte, the even K index in the low nibble;
 *   scales u8 [G][R][4]:  the scale byte of block b of row r sits at
 *          [b / 4][r][b % 4].
 * Blocks of a last, partial stage past K / 32 have zero codes and zero scale
 * bytes (the quantisers write them; inputs from elsewhere must hold zeros).
 * One GEMM stage of a row tile is then one contiguous run of each operand.
 *
 * This departs from the plain row-major contract (codes [R][K/2], scales
 * [R][K/32]) that an MXFP4 interface would otherwise expose: every prepare
 * output and every weight here is stage-major. The reason is measured GEMM
 * time on MI355X: with row-major scales each 128-entry stage of a 128-row
 * tile gathers 128 separate 4-byte scale runs, and with row-major codes 128
 * separate 64-byte code runs; stage-major scales made the two-path GEMM
 * 11-17% faster and stage-major codes another 5-9%. The canonical layout
 * stays available at the boundary: sharq_pack_stage_major and
 * sharq_unpack_stage_major convert in both directions without changing any
 * byte, so a caller holding canonical tensors packs them once (weights) or
 * unpacks prepare's output when it needs row-major codes.
 *
 * Conventions for every entry point below:
 *  - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *    every buffer; the library allocates nothing and keeps no state, so calls
 *    are re-entrant.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *  - Arguments are validated on the host before any HIP call. Errors return a
 *    negative sharq_status and enqueue nothing. A fault inside a kernel shows
 *    up at the caller's next synchronisation (the HIP convention).
 *  - A call with no rows (T, P or O equal to 0) is a no-op that returns
 *    SHARQ_OK once the shape arguments are valid; its pointers may be NULL.
 *  - Inputs must be finite; with NaN or Inf the outputs are unspecified.
 *  - Activations and outputs are row-major; sizes are element counts.
 *    T = rows (tokens), K = input features, O = output features.
 *  - Alignment: every pointer 16-byte aligned; ldx a multiple of 8.
 */
#ifndef SHARQ_H
#define SHARQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef SHARQ_API
#define SHARQ_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SHARQ_OK = 0,
  SHARQ_EINVAL = -1,       /* bad shape, stride or NULL pointer */
  SHARQ_EALIGN = -2,       /* pointer not 16-byte aligned, or ldx % 8 != 0 */
  SHARQ_EUNSUPPORTED = -3, /* (n, m) not in {(2,4), (8,16)} */
  SHARQ_EHIP = -4,         /* the HIP launch itself failed */
  SHARQ_ENOTIMPL = -5,     /* a shape class this library does not handle */
  SHARQ_ESCRATCH = -6      /* needs more scratch than SHARQ_SCRATCHFREE_MAX_BYTES */
} sharq_status;

/* Host. Static string describing a status code; never NULL. */
SHARQ_API const char* sharq_status_string(int status);

/* Host. Version of this ABI (bumped on any signature or layout change). */
SHARQ_API int sharq_abi_version(void);

/*
 * sharq_prepare -- the fused prepare operator (SharQ page, Abstract: mask
 * generation, residual construction and layer-norm absorption in one
 * operator; Section 1: the residual is taken against the quantised backbone).
 *
 *  x        bf16 [T][ldx], the first K entries of each row are used.
 *  gamma    bf16 [K] RMSNorm weight absorbed as x' = x * gamma (fp32), or NULL;
 *           K entries are read, so it must hold at least K (the library cannot
 *           check the length of a device buffer).
 *  n, m     N:M pattern: (2,4) or (8,16). Selection keeps, in each group of m
 *           consecutive K entries, the n largest |x'|; equal |x'| go to the
 *           lower index.
 *  bb_codes   u8 [G][T][64] backbone E2M1 codes (0x0 at dropped positions)
 *  bb_scales  u8 [G][T][4]  backbone E8M0 scales, stage-major
 *  res_codes  u8 [G][T][64] residual codes, residual r = x' - dequant(backbone)
 *  res_scales u8 [G][T][4]  residual scales, stage-major
 *  mask       u8 [T][K/8]   bit (k & 7) of byte k >> 3 set when k is kept, or
 *                           NULL to skip writing it.
 * Requires K % 32 == 0, K % m == 0, T >= 0 (T == 0 is a no-op), ldx >= K,
 * T * K / 32 < 2^31.
 */
SHARQ_API int sharq_prepare(const uint16_t* x, int64_t T, int64_t K, int64_t ldx,
                  const uint16_t* gamma, int n, int m,
                  uint8_t* bb_codes, uint8_t* bb_scales,
                  uint8_t* res_codes, uint8_t* res_scales,
                  uint8_t* mask, hipStream_t stream);

/*
 * sharq_prepare_rms -- sharq_prepare with the whole RMSNorm absorbed (SharQ
 * page, Abstract: the fused prepare operator absorbs the layer norm): per row
 *   r = fp32(1 / sqrt(S / K + eps)),  x_n = bf16_rne(fp32(x) * r),
 *   x' = x_n * gamma (fp32; gamma may be NULL),
 * then the prepare operator on x'. S, the row's sum of squares, is summed in
 * float64 in a fixed order: the 32 squares of each MX block one after the
 * other in index order, then the block sums by a pairwise tree over blocks in
 * index order (adjacent pairs, level by level, padded with zero blocks to a
 * power of two); mean, eps, sqrt and reciprocal are correctly rounded float64
 * operations. One kernel runs: x is read from HBM once and the scale r of a
 * row is formed before its blocks are coded.
 *  eps        > 0 and finite.
 *  gamma      bf16 [K] or NULL, K entries read (as sharq_prepare).
 *  rms_scale  fp32 [T], written with r (required).
 *  other arguments as sharq_prepare. Requires K / 32 <= 4096
 *  (SHARQ_ENOTIMPL otherwise).
 */
SHARQ_API int sharq_prepare_rms(const uint16_t* x, int64_t T, int64_t K, int64_t ldx,
                      const uint16_t* gamma, float eps, int n, int m, float* rms_scale,
                      uint8_t* bb_codes, uint8_t* bb_scales,
                      uint8_t* res_codes, uint8_t* res_scales,
                      uint8_t* mask, hipStream_t stream);

/*
 * sharq_quantize_mxfp4 -- plain MXFP4 of bf16 rows along K (no mask, no
 * residual), the same element and scale rules as sharq_prepare. Used to
 * produce the pre-quantised weight [O][K] that sharq_linear reads.
 *  x bf16 [T][ldx]; codes u8 [G][T][64]; scales u8 [G][T][4] (stage-major).
 * Requires K % 32 == 0, ldx >= K, T * K / 32 < 2^31.
 */
SHARQ_API int sharq_quantize_mxfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx,
                         uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * sharq_linear -- the two-path FP4 GEMM (SharQ page, Abstract: a sparse FP4
 * GEMM on the backbone and a dense FP4 GEMM on the residual share one FP4
 * weight load; Section 1: the residual path accumulates into the sparse
 * output):
 *   Y[t][o] = sum_k deq(bb)[t][k] * deq(W)[o][k] + sum_k deq(res)[t][k] * deq(W)[o][k]
 *  bb_codes/res_codes u8 [G][T][64], bb_scales/res_scales u8 [G][T][4] (as
 *  written by sharq_prepare); w_codes u8 [G][O][64], w_scales u8 [G][O][4]
 *  (as written by sharq_quantize_mxfp4); y fp32 [T][ldy], overwritten (not
 *  accumulated into).
 * Accumulation is fp32 in an unspecified order. Requires K % 32 == 0,
 * ldy >= O, T >= 0 (T == 0 or O == 0 is a no-op).
 */
SHARQ_API int sharq_linear(const uint8_t* bb_codes, const uint8_t* bb_scales,
                 const uint8_t* res_codes, const uint8_t* res_scales,
                 const uint8_t* w_codes, const uint8_t* w_scales,
                 int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                 hipStream_t stream);

/*
 * sharq_linear_workspace_bytes -- host. Bytes of device workspace with which
 * sharq_linear_ws splits K for a (T, O, K) problem, or 0 when it would not
 * split (then sharq_linear_ws needs no workspace). Invalid shapes give 0.
 * The split count is the one of 1 .. 16 with the smallest estimated launch
 * time on MI355X (K loop, weight streaming, partials' traffic); it depends
 * on the shape only.
 */
SHARQ_API int64_t sharq_linear_workspace_bytes(int64_t T, int64_t O, int64_t K);

/*
 * sharq_linear_ws -- sharq_linear (same arguments, same result up to the
 * accumulation order) that may split K across workgroups when the output has
 * too few tiles to fill the GPU and K is long enough to pay for it (decode
 * and mid-sized T, narrow layers). Each split
 * writes its fp32 partial tile into the workspace and a second kernel sums
 * the partials in split order, so calls are deterministic.
 *  workspace  device memory of at least sharq_linear_workspace_bytes(T, O, K)
 *             bytes, 16-byte aligned; its contents need no initialisation
 *             and are overwritten. Calls that may overlap in time need
 *             separate workspaces. With NULL or a smaller workspace the call
 *             runs exactly as sharq_linear.
 */
SHARQ_API int sharq_linear_ws(const uint8_t* bb_codes, const uint8_t* bb_scales,
                    const uint8_t* res_codes, const uint8_t* res_scales,
                    const uint8_t* w_codes, const uint8_t* w_scales,
                    int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                    void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * sharq_linear_scratchfree -- sharq_linear_ws without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments and result as sharq_linear, bit-identical to
 * sharq_linear_ws with a large enough workspace (the same split plan and
 * kernels).
 *
 * The split-K partials live in a static device array of
 * SHARQ_SCRATCHFREE_MAX_BYTES bytes that every GPU the library runs on holds
 * from load until the process ends. Every call on one GPU shares that GPU's
 * array: calls that may overlap in time on one GPU (several streams or host
 * threads) race and give undefined results; serialise them. The array's
 * contents need no initialisation (each call writes every partial it reads).
 *
 * Errors: as sharq_linear; SHARQ_ESCRATCH, before any HIP call, when the
 * split plan needs more than SHARQ_SCRATCHFREE_MAX_BYTES
 * (sharq_linear_workspace_bytes(T, O, K) tells how much it needs). The first
 * call on a device looks up the array's device address (no allocation).
 */
#define SHARQ_SCRATCHFREE_MAX_BYTES ((int64_t)32 << 20)
SHARQ_API int sharq_linear_scratchfree(const uint8_t* bb_codes, const uint8_t* bb_scales,
                             const uint8_t* res_codes, const uint8_t* res_scales,
                             const uint8_t* w_codes, const uint8_t* w_scales,
                             int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                             hipStream_t stream);

/*
 * sharq_linear_grouped -- sharq_linear per expert segment, for mixture-of-
 * experts layers (SharQ page, Abstract: MoE models are among the targets).
 * Output row p (0 <= p < P) belongs to the expert e with
 * seg_offsets[e] <= p < seg_offsets[e+1]; it reads activation row a_rows[p]
 * (or row p when a_rows is NULL) and expert e's weight.
 *  bb_codes/res_codes u8 [G][T_src][64], bb_scales/res_scales u8 [G][T_src][4]
 *              the prepared activation rows (T_src >= P when a_rows is NULL).
 *  a_rows      i32 [P] device, each in [0, T_src), or NULL.
 *  seg_offsets i32 [E+1] device, non-decreasing, [0] = 0, [E] = P.
 *  w_codes u8 [E][G][O][64], w_scales u8 [E][G][O][4] (each expert's
 *              tensor stage-major); y fp32 [P][O].
 * Segment and gather contents are read on the device: segment bounds are
 * clamped to [0, P] (an empty or reversed segment has no rows), and a
 * gathered row outside [0, T_src) reads as zeros, so malformed contents give
 * unspecified values but no access outside the buffers.
 * SHARQ_EINVAL also when (ceil(P/128) + E) * ceil(O/256), the bound on the
 * number of 128 x 256 tiles, exceeds 2^24.
 */
SHARQ_API int sharq_linear_grouped(const uint8_t* bb_codes, const uint8_t* bb_scales,
                         const uint8_t* res_codes, const uint8_t* res_scales,
                         int64_t T_src, const int32_t* a_rows,
                         const int32_t* seg_offsets, int32_t E,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t P, int64_t O, int64_t K, float* y,
                         hipStream_t stream);

/*
 * sharq_linear_silu_prepare -- a fused gate|up projection of a gated MLP:
 * the two-path FP4 GEMM of sharq_linear against a weight whose 2I rows are
 * the gate rows (0 .. I-1) followed by the up rows (I .. 2I-1), then
 *   h[t][i] = bf16(silu(Y[t][i]) * Y[t][I + i])      (as sharq_silu_mul)
 * and then the prepare operator on h (as sharq_prepare with no gamma), so
 * that h never round-trips through HBM in fp32 (glue around the method; the
 * two-path GEMM and the prepare are the SharQ page's, Abstract and
 * Section 1).
 *  bb_codes/res_codes u8 [G][T][64], bb_scales/res_scales u8 [G][T][4]: the
 *              prepared input rows (G = K / 128);
 *  w_codes u8 [G][2I][64], w_scales u8 [G][2I][4]: the fused weight;
 *  h           bf16 [T][I] or NULL;
 *  h_bb_codes, h_res_codes u8 [I/128][T][64], h_bb_scales, h_res_scales
 *              u8 [I/128][T][4], h_mask u8 [T][I/8] (or NULL): prepare(h)
 *              with pattern n:m, or all four NULL (then h must be given).
 * Outputs are bit-identical to sharq_linear + sharq_silu_mul + sharq_prepare
 * run one after the other. Requires I % 128 == 0 and K % 128 == 0
 * (SHARQ_ENOTIMPL otherwise), T * K / 2 < 2^31 and I * K < 2^31.
 */
SHARQ_API int sharq_linear_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales,
                              const uint8_t* res_codes, const uint8_t* res_scales,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              int64_t T, int64_t I, int64_t K, int n, int m,
                              uint16_t* h, uint8_t* h_bb_codes, uint8_t* h_bb_scales,
                              uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask,
                              hipStream_t stream);

/*
 * sharq_linear_silu_prepare_workspace_bytes -- host. Bytes of device
 * workspace with which sharq_linear_silu_prepare_ws splits K for a (T, I, K)
 * problem (gate|up weight of 2 I rows), or 0 when it would not split: the
 * plan of sharq_linear_workspace_bytes(T, 2 I, K) (the fused kernel has the
 * plain GEMM's row tiles, the 32- and 64-row decode tiles included). Invalid
 * shapes give 0.
 */
SHARQ_API int64_t sharq_linear_silu_prepare_workspace_bytes(int64_t T, int64_t I, int64_t K);

/*
 * sharq_linear_silu_prepare_ws -- sharq_linear_silu_prepare that may split K
 * across workgroups where its plan splits (too few output tiles to fill the
 * GPU, K long enough): the gate|up GEMM stores fp32 partials over K slices in
 * `workspace`, and one more kernel sums them in slice order, forms h and
 * codes prepare(h) (glue and prepare as in sharq_linear_silu_prepare; the
 * method is the SharQ page's, Abstract and Section 1).
 *  arguments as sharq_linear_silu_prepare, plus
 *  workspace, workspace_bytes: caller-owned device memory of at least
 *              sharq_linear_silu_prepare_workspace_bytes(T, I, K) bytes,
 *              16-byte aligned; contents need no initialisation and are
 *              overwritten. With a smaller (or NULL) workspace, or when that
 *              function returns 0, this is sharq_linear_silu_prepare.
 * Outputs are bit-identical to sharq_linear_ws (T, 2 I, K) + sharq_silu_mul
 * + sharq_prepare (the same split plan). Errors: as
 * sharq_linear_silu_prepare; workspace_bytes < 0, or > 0 with a NULL
 * workspace, is SHARQ_EINVAL; a misaligned workspace SHARQ_EALIGN.
 */
SHARQ_API int sharq_linear_silu_prepare_ws(const uint8_t* bb_codes, const uint8_t* bb_scales,
                              const uint8_t* res_codes, const uint8_t* res_scales,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              int64_t T, int64_t I, int64_t K, int n, int m,
                              uint16_t* h, uint8_t* h_bb_codes, uint8_t* h_bb_scales,
                              uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask,
                              void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * sharq_linear_grouped_silu_prepare -- the fused gate|up projection of
 * sharq_linear_silu_prepare per expert segment, with the segments, the row
 * gather and the per-expert weights of sharq_linear_grouped (mixture-of-
 * experts layers: SharQ page, Abstract). Output row p is sorted pair p.
 *  bb_codes .. res_scales, T_src, a_rows, seg_offsets, E: as for
 *              sharq_linear_grouped;
 *  w_codes u8 [E][G][2I][64], w_scales u8 [E][G][2I][4]: each expert's
 *              fused weight (gate rows 0 .. I-1, up rows I .. 2I-1);
 *  h           bf16 [P][I] or NULL;
 *  h_bb_codes, h_res_codes u8 [I/128][P][64], h_bb_scales, h_res_scales
 *              u8 [I/128][P][4], h_mask u8 [P][I/8] (or NULL): prepare(h)
 *              with pattern n:m, or all four NULL (then h must be given).
 * Outputs are bit-identical to sharq_linear_grouped + sharq_silu_mul +
 * sharq_prepare. Requires I % 128 == 0 and K % 128 == 0 (SHARQ_ENOTIMPL
 * otherwise), T_src * K / 2 < 2^31 and I * K < 2^31 (SHARQ_ENOTIMPL);
 * SHARQ_EINVAL when (ceil(P/128) + E) * I / 128 exceeds 2^24.
 */
SHARQ_API int sharq_linear_grouped_silu_prepare(const uint8_t* bb_codes, const uint8_t* bb_scales,
                              const uint8_t* res_codes, const uint8_t* res_scales,
                              int64_t T_src, const int32_t* a_rows,
                              const int32_t* seg_offsets, int32_t E,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              int64_t P, int64_t I, int64_t K, int n, int m,
                              uint16_t* h, uint8_t* h_bb_codes, uint8_t* h_bb_scales,
                              uint8_t* h_res_codes, uint8_t* h_res_scales, uint8_t* h_mask,
                              hipStream_t stream);

/*
 * Compressed sparse backbone -- the "sparse input compression" of the fused
 * prepare (SharQ page, Abstract; the page gives no format). For N:M with
 * N = M / 2 (2:4 and 8:16) a row's backbone keeps, per group of M, only its N
 * kept codes in index order (K / 4 bytes instead of K / 2), plus one field
 * per group: the colexicographic rank of the kept positions,
 * C(c_1, 1) + ... + C(c_N, N) for kept c_1 < ... < c_N inside the group, in
 * ceil(log2 C(M, N)) bits (3 for 2:4, 14 for 8:16: the 0.75 and 0.875 bits
 * per element of the 8:16 page, abstract). A row's fields are a bit stream,
 * group g at bits [g b, g b + b), least significant bit first. Block scales
 * (bb_scales) are unchanged and not touched. All shapes need K % 64 == 0
 * (SHARQ_ENOTIMPL otherwise).
 *
 * sharq_backbone_meta_row_bytes -- host: bytes of one row's field stream,
 * K / 64 * 6 (2:4) or K / 64 * 7 (8:16); a negative status on bad arguments.
 */
SHARQ_API int64_t sharq_backbone_meta_row_bytes(int64_t K, int n, int m);

/*
 * sharq_compress_backbone -- the compressed form of a prepared backbone.
 *  bb_codes u8 [G][T][64] (stage-major, as written by sharq_prepare) and
 *  mask u8 [T][K/8] (required: it names the kept positions);
 *  codes u8 [T][K/4] (row-major, two codes per byte, earlier in the low
 *  nibble), meta u8 [T][sharq_backbone_meta_row_bytes(K, n, m)].
 * Precondition: exactly N mask bits per group and code 0 at dropped
 * positions (what sharq_prepare writes); otherwise the output is unspecified
 * (no access leaves the buffers). Pointers 16-byte aligned except meta.
 */
SHARQ_API int sharq_compress_backbone(const uint8_t* bb_codes, const uint8_t* mask,
                              int64_t T, int64_t K, int n, int m,
                              uint8_t* codes, uint8_t* meta, hipStream_t stream);

/*
 * sharq_expand_backbone -- the inverse: codes and meta as above -> the dense
 * stage-major bb_codes [G][T][64] (blocks of a last, partial stage are
 * written as zero) and the mask [T][K/8] (or NULL to skip it). Fields of
 * C(M, N) or more give unspecified codes and mask, still inside the buffers.
 */
SHARQ_API int sharq_expand_backbone(const uint8_t* codes, const uint8_t* meta,
                              int64_t T, int64_t K, int n, int m,
                              uint8_t* bb_codes, uint8_t* mask, hipStream_t stream);

/*
 * sharq_moe_combine -- the weighted combine of a mixture-of-experts layer
 * (glue around sharq_linear_grouped, not part of the method; the SharQ
 * page, Abstract, names MoE models among the targets):
 *   out[t][c] = sum_{j = 0 .. k-1, pair_index[t][j] >= 0} weights[t][j] * y[pair_index[t][j]][c]
 * accumulated in fp32 in slot order j = 0, 1, ... with one fused
 * multiply-add per slot (deterministic).
 *  y           fp32 [P][H], the grouped GEMM's output rows (sorted pairs);
 *  pair_index  i32 [T][k], the pairs of token t (-1: empty slot; an index
 *              outside [0, P) is treated as an empty slot);
 *  weights     fp32 [T][k];
 *  out         fp32 [T][H] or NULL; out_bf16 bf16 [T][H] (the fp32 sum
 *              rounded to nearest even) or NULL; at least one is given.
 * Requires H % 4 == 0 and 1 <= k <= 64; y and out 16-byte aligned, out_bf16
 * 8-byte aligned, pair_index and weights 4-byte aligned.
 */
SHARQ_API int sharq_moe_combine(const float* y, int64_t P, int64_t H,
                              const int32_t* pair_index, const float* weights,
                              int64_t T, int32_t k, float* out, uint16_t* out_bf16,
                              hipStream_t stream);

/*
 * sharq_silu_mul -- glue between a fused gate|up projection and the down
 * projection (not part of the method): h[t][i] = bf16(silu(g) * u) with
 * g = gu[t][i], u = gu[t][I + i], silu(g) = g / (1 + exp(-g)), fp32 math,
 * round-to-nearest-even to bf16.
 *  gu fp32 [T][2I]; h bf16 [T][I]. Requires I % 8 == 0.
 */
SHARQ_API int sharq_silu_mul(const float* gu, int64_t T, int64_t I, uint16_t* h,
                   hipStream_t stream);

/*
 * sharq_pack_stage_major / sharq_unpack_stage_major -- layout conversion
 * (data movement only) between the canonical row-major block-FP4 layout an
 * external quantiser writes and the stage-major layout of every other entry
 * point:
 *   row-major:   codes u8 [R][K/2] (even K index in the low nibble),
 *                scales u8 [R][K/block] (one byte per block of entries);
 *   stage-major: codes u8 [G][R][64], scales u8 [G][R][128/block],
 *                G = ceil(K/128), bytes past K zero (packing writes them).
 * block is 32 (MXFP4, E8M0 scales) or 16 (NVFP4, E4M3 scales). Every code
 * and scale byte is kept unchanged. Requires K % 32 == 0 and
 * G * R * 64 < 2^31 (SHARQ_EINVAL otherwise); code pointers 16-byte aligned
 * (scale pointers may have any alignment). Unpacking writes only the K/2
 * code bytes and K/block scale bytes of each row.
 */
SHARQ_API int sharq_pack_stage_major(const uint8_t* codes_rm, const uint8_t* scales_rm,
                           int64_t R, int64_t K, int block,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);
SHARQ_API int sharq_unpack_stage_major(const uint8_t* codes, const uint8_t* scales,
                             int64_t R, int64_t K, int block,
                             uint8_t* codes_rm, uint8_t* scales_rm, hipStream_t stream);

/*
 * NVFP4 (SharQ page, Abstract: the method generalises to NVFP4 as well as
 * MXFP4). The pages name NVFP4 without defining it; its public definition is
 * used: E2M1 codes in blocks of 16 consecutive K entries, one FP8 E4M3
 * (OCP E4M3FN) scale byte per block, one fp32 scale per tensor, so an entry
 * decodes to e2m1(code) * e4m3(scale byte) * tensor_scale. Coding of a block
 * (fp32, round to nearest even): v = amax / fp32(6 * tensor_scale); scale =
 * the E4M3 value nearest to v (ties to the even code, 448 above 448);
 * d = fp32(e4m3(scale) * tensor_scale); code = E2M1 code nearest to
 * fp32(x / d), saturated at 6, sign kept on zero (all signed zeros if d == 0).
 * Layout: stage-major as above with codes u8 [G][R][64] (the same byte and
 * nibble positions) and scales u8 [G][R][8]: the E4M3 byte of 16-block j of
 * stage g of row r at [g][r][j]. Bytes past K are zero.
 * tensor_scale must be finite and > 0 (SHARQ_EINVAL otherwise); the usual
 * choice is amax / (6 * 448) of the tensor (a calibration the caller makes).
 */

/*
 * sharq_prepare_nvfp4 -- sharq_prepare with NVFP4 codes. The activation has
 * one tensor scale shared by backbone and residual (each has its own block
 * scales). The residual is r = fp32(x' - fp32(e2m1 * e4m3 * tensor_scale)).
 *  bb_codes, res_codes    u8 [G][T][64]
 *  bb_scales, res_scales  u8 [G][T][8] (E4M3 bytes)
 *  gamma                  bf16 [K] or NULL, K entries read (as sharq_prepare).
 *  other arguments and requirements as sharq_prepare.
 */
SHARQ_API int sharq_prepare_nvfp4(const uint16_t* x, int64_t T, int64_t K, int64_t ldx,
                        const uint16_t* gamma, int n, int m, float tensor_scale,
                        uint8_t* bb_codes, uint8_t* bb_scales,
                        uint8_t* res_codes, uint8_t* res_scales,
                        uint8_t* mask, hipStream_t stream);

/*
 * sharq_quantize_nvfp4 -- NVFP4 of a bf16 weight w [O][ldw] (first K entries
 * of each row) with tensor scale tensor_scale: codes u8 [G][O][64], scales
 * u8 [G][O][8]. Requirements as sharq_quantize_mxfp4.
 */
SHARQ_API int sharq_quantize_nvfp4(const uint16_t* w, int64_t O, int64_t K, int64_t ldw,
                         float tensor_scale, uint8_t* codes, uint8_t* scales,
                         hipStream_t stream);

/*
 * sharq_linear_nvfp4 -- the two-path GEMM on NVFP4 operands:
 *   Y = deq(A_s) deq(W)^T + deq(A_r) deq(W)^T   (fp32 accumulation),
 * A_s, A_r with tensor scale a_tensor_scale, W with w_tensor_scale.
 * The codes are widened to fp16 (code * block scale is exact there) and
 * multiplied on the fp16 matrix cores.
 *  bb_*, res_*   as written by sharq_prepare_nvfp4 ([G][T][64], [G][T][8]);
 *  w_codes u8 [G][O][64], w_scales u8 [G][O][8];  y fp32 [T][ldy].
 * Requires K % 32 == 0, ldy >= O, ceil(T/128) * ceil(O/256) <= 2^24.
 */
SHARQ_API int sharq_linear_nvfp4(const uint8_t* bb_codes, const uint8_t* bb_scales,
                       const uint8_t* res_codes, const uint8_t* res_scales,
                       float a_tensor_scale, const uint8_t* w_codes,
                       const uint8_t* w_scales, float w_tensor_scale,
                       int64_t T, int64_t O, int64_t K, float* y, int64_t ldy,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H */
