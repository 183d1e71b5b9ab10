/*
 * fp8blk -- block-scaled ("fine-grained") FP8 linear layer for AMD MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Weights are stored as 8-bit floats with one fp32 scale per 2D block of
 * 128x128, and activations are quantized at run time with one fp32 scale per
 * token and per group of 128 input channels, the group matching the weight
 * block along the input channel ("Fine-grained FP8" page of the transformers
 * docs, introduction; run-time activation scales are the "dynamic"
 * activation scheme of its "DeepGEMM fast path" section; fp32 is the default
 * scale type, per its "UE8M0 scale format" section).  The linear layer's
 * value is that of dequantize-then-matmul ("BFL (fp8r / nvfp4)" page of the
 * diffusers docs, "Kernels").
 *
 * The readings this library fixes where the pages are silent:
 *   - the 8-bit format is OCP FP8 E4M3FN (bias 7, max 448, no infinities);
 *   - scale s = fl32(amax / 448) over the block or group (s is the
 *     dequantization multiplier: x ~= dec(q) * s);
 *   - code q = E4M3(fl32(x / s)): the IEEE fp32 quotient is rounded first,
 *     then rounded to nearest-even E4M3 and saturated to +-448;
 *   - an all-zero block or group gets s = 0 and signed-zero codes;
 *   - y[m,n] = bf16_RNE( sum_kb x_s[m,kb] * w_s[n/128,kb] *
 *                        sum_{k in block kb} dec(x_q[m,k]) * dec(w_q[n,k]) ),
 *     with fp32 accumulation; the 128-long inner sums run on fp8 matrix
 *     cores and the scale pair is applied once per K block.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   - All tensor pointers are DEVICE pointers; the caller owns every buffer.
 *     The library never allocates, frees or keeps a pointer; it is stateless
 *     apart from a per-device architecture check that is cached.
 *   - Layouts are dense row-major: x [M,K], W [N,K] (the nn.Linear layout,
 *     K contiguous), x_s [M, K/128], w_s [ceil(N/128), K/128], y [M,N].
 *     bf16 tensors are raw 16-bit patterns; E4M3 codes are bytes.
 *   - K must be a positive multiple of 128.  N and M may be any size >= 0;
 *     a last weight block row with fewer than 128 rows covers only the rows
 *     that exist.  M == 0 or N == 0 (or E == 0) is a no-op returning OK.
 *   - Every tensor base pointer must be 16-byte aligned (expert_offsets:
 *     and expert_counts: 4-byte aligned, as int32 arrays; a single static scale: 4-byte
 *     aligned; E8M0 scale-byte arrays: any address).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Inputs must stay valid until the stream reaches the launch.
 *     Outputs must not alias inputs.
 *   - Arguments are validated before any HIP runtime call, in the order
 *     null pointers, shapes, alignment; then the current device must be a
 *     gfx950, else FP8BLK_ERR_DEVICE.  A failed launch returns
 *     FP8BLK_ERR_LAUNCH.  Faults inside a kernel surface as HIP errors at
 *     the caller's next synchronisation.
 *   - Non-finite inputs (NaN, Inf) are outside the contract: results are
 *     unspecified, but the kernels stay in bounds.
 *   - Size limits: M, N <= 2^31 - 1 and K <= 2^24 per call.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FP8BLK_API __attribute__((visibility("default")))
#else
#define FP8BLK_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8BLK_OK = 0,
    FP8BLK_ERR_NULL = 1,    /* a required pointer is NULL                    */
    FP8BLK_ERR_SHAPE = 2,   /* negative size, K % 128 != 0, size over limit  */
    FP8BLK_ERR_ALIGN = 3,   /* a base pointer is not 16-byte aligned         */
    FP8BLK_ERR_DEVICE = 4,  /* no device, or the current device is not gfx950 */
    FP8BLK_ERR_LAUNCH = 5,  /* the kernel launch failed                      */
    FP8BLK_ERR_SCRATCH = 6  /* more device scratch needed than the library holds */
} fp8blk_status;

#define FP8BLK_BLOCK 128
#define FP8BLK_ABI_VERSION 1

/* Weight quantization, one fp32 scale per 128x128 block.
 * "Fine-grained FP8" page, introduction: weights are brought to 8 bits per
 * 2D block, weight_block_size = (128, 128).  Done once, when weights load.
 *   w_bf16  [N,K] bf16 in
 *   w_q     [N,K] E4M3 codes out
 *   w_scale [ceil(N/128), K/128] fp32 out; block (nb,kb) covers rows
 *           [128nb, min(N,128nb+128)) and columns [128kb, 128kb+128). */
FP8BLK_API fp8blk_status fp8_weight_block_quant(const void *w_bf16, int64_t N, int64_t K,
                                                void *w_q, float *w_scale, void *stream);

/* Dynamic activation quantization, one fp32 scale per token per 128 input
 * channels.  "Fine-grained FP8" page, introduction (per token, per group,
 * the group matching the weights' input-channel block, 128 by default) and
 * "DeepGEMM fast path" (activation_scheme = "dynamic": scales are computed
 * on every call).
 *   x_bf16  [M,K] bf16 in
 *   x_q     [M,K] E4M3 codes out
 *   x_scale [M, K/128] fp32 out; group (m,g) covers columns [128g, 128g+128). */
FP8BLK_API fp8blk_status fp8_act_quant_group(const void *x_bf16, int64_t M, int64_t K,
                                             void *x_q, float *x_scale, void *stream);

/* Block-scaled FP8 GEMM, y = x * W^T in bf16.  "Fine-grained FP8" page,
 * "DeepGEMM fast path": the FP8 linear layer with (128,128) weight blocks
 * and dynamic activation groups; value as dequantize-then-matmul ("BFL"
 * page, "Kernels").  The scale pair x_scale[m,kb] * w_scale[n/128,kb] is
 * applied to each 128-long partial sum inside the K loop.
 *   x_q [M,K], x_scale [M,K/128], w_q [N,K], w_scale [ceil(N/128),K/128] in
 *   y_bf16 [M,N] out (bf16, round to nearest even). */
FP8BLK_API fp8blk_status fp8_block_gemm(const void *x_q, const float *x_scale,
                                        const void *w_q, const float *w_scale,
                                        int64_t M, int64_t N, int64_t K,
                                        void *y_bf16, void *stream);

/* The same GEMM with a caller workspace, for shapes whose grid of output
 * tiles would leave compute units idle: small M and N with long K (e.g.
 * the DeepSeek-V3 q_a and kv_a projections at a few hundred tokens); large
 * grids of 256x256 tiles whose last round of 256 compute units is partly
 * empty (e.g. 8192 x 7168 x 16384: 896 tiles, 3.5 rounds), or that fill
 * less than one round with long K (e.g. 512 x 7168 x 16384); and decode
 * batches of 9 to 16 rows with long K (e.g. a 4096 x 14336 down
 * projection), where a workgroup covering 64 output columns over part of K
 * re-reads less of x than one covering 16 columns over all of it, and of
 * 33 to 64 rows with K >= 6144, where one row tile of 128 split over K
 * beats the decode kernel's per-workgroup re-reads of x.  The same
 * operation and passage as fp8_block_gemm: a workgroup runs one output tile
 * over one contiguous range of K blocks, promoting each 128-long partial
 * sum with its scale pair into fp32 as fp8_block_gemm does, and stores the
 * range's unrounded fp32 sums in the workspace; a second kernel adds a
 * tile's ranges in K order and rounds once to bf16.  In the partly empty
 * last round case only that round's tiles are split (their K blocks cut
 * into 256 equal ranges, "stream-K"); the whole rounds before it run
 * unsplit in the same launch.  The result meets the same tolerance; split
 * tiles are not bit-identical to fp8_block_gemm (the fp32 sums are
 * associated differently), unsplit ones are.
 *   fp8_block_gemm_workspace_bytes(M, N, K): bytes the split needs, 0 when
 *     it is not used for these sizes.  17 <= M <= 32 never splits.  M > 32
 *     (with K >= 6144 when M <= 64):
 *     either at most 128 output tiles of 128x128 and K long enough for the
 *     split to gain (a time model measured on MI355X picks the number of K
 *     ranges, 2 to min(256 / tiles, K / 512), or none): ranges x M x N x 4
 *     bytes; or at least 192 tiles of 256x256, not a whole number of rounds
 *     of 256, where a time model (1.9 us per K block of a tile against the
 *     partial sums' traffic) gains more than 8 us: (the ranges, at most
 *     256, plus the last round's tiles) x 256 KB (100.7 MB for 8192 x 7168
 *     x 16384); or 32 to 191 tiles of 256x256 with K >= 7168 and more than
 *     128 tiles of 128x128, run wholly as stream-K where the same model
 *     beats an estimate of the 128x128 kernels by 10 % (e.g. the
 *     DeepSeek-V3 o_proj, MLP up and MLP down at M = 512): (the ranges plus
 *     the tiles) x 256 KB (81.8 MB for 512 x 7168 x 16384).
 *     9 <= M <= 16: ceil(N / 64) column groups times the number of K ranges
 *     (at most 256 / groups and K / 2048) must reach 192, where N is too
 *     small for ceil(N / 64) groups alone to fill the chip and K is at most
 *     65536.  Invalid sizes: 0.  Host arithmetic only, no HIP call.
 *   fp8_block_gemm_ws: arguments as fp8_block_gemm, plus `workspace`
 *     (device, 16-byte aligned, owned by the caller, overwritten, not
 *     initialised by the caller) of `workspace_bytes` bytes.  When the
 *     workspace is NULL or smaller than fp8_block_gemm_workspace_bytes(M,
 *     N, K), or that is 0, the call is exactly fp8_block_gemm (bit-identical
 *     output) and the workspace is not touched.  Calls that share a
 *     workspace must be ordered on one stream.  Errors as fp8_block_gemm;
 *     a misaligned workspace that would be used is FP8BLK_ERR_ALIGN. */
FP8BLK_API size_t fp8_block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
FP8BLK_API fp8blk_status fp8_block_gemm_ws(const void *x_q, const float *x_scale,
                                           const void *w_q, const float *w_scale,
                                           int64_t M, int64_t N, int64_t K, void *y_bf16,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/* fp8_block_gemm_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, plan and kernels as
 * fp8_block_gemm_ws given a large enough workspace (bit-identical output),
 * except that shapes fp8_block_gemm_ws would give the stream-K split of a
 * partly empty last round run unsplit, as fp8_block_gemm (bit-identical to
 * it; those partial sums take up to ~100 MB); the split's fp32 partial sums
 * go to a device array inside the library
 * of FP8BLK_SCRATCH_BYTES bytes, one per GPU, held until the process ends,
 * whose address is looked up once per device on the first call made with
 * that device current.  Allocates nothing.
 *   Arguments and errors as fp8_block_gemm; FP8BLK_ERR_SCRATCH if the split
 *   would need more than FP8BLK_SCRATCH_BYTES (no valid size does today:
 *   the largest plan is 16 MiB plus a few bytes).
 *   All calls on one GPU share its scratch array, which keeps the last
 *   call's contents (the split writes every partial it reads, so nothing
 *   needs clearing): calls that may overlap on one GPU (different streams,
 *   no ordering between them) race on it and must be serialised by the
 *   caller. */
#define FP8BLK_SCRATCH_BYTES ((size_t)16 * 1024 * 1024 + (size_t)64 * 1024)
FP8BLK_API fp8blk_status fp8_block_gemm_noalloc(const void *x_q, const float *x_scale,
                                                const void *w_q, const float *w_scale,
                                                int64_t M, int64_t N, int64_t K,
                                                void *y_bf16, void *stream);

/* Grouped block-scaled FP8 GEMM for mixture-of-experts layers: expert e
 * multiplies rows [off[e], off[e+1]) of x by its own W[e].  "Fine-grained
 * FP8" page, "UE8M0 scale format": expert matmuls run through grouped
 * back-ends that take fp32 scales directly; "DeepGEMM fast path" names the
 * expert back-ends.
 *   x_q [total_M,K], x_scale [total_M,K/128]
 *   w_q [E,N,K], w_scale [E, ceil(N/128), K/128]
 *   expert_offsets: DEVICE int32 [E+1], non-decreasing, off[0] = 0,
 *       off[E] <= total_M.  Trusted (read on the device, no host sync);
 *       row ranges are clamped to [0, total_M).
 *   y_bf16 [total_M,N] out; rows that belong to no expert are not written. */
FP8BLK_API fp8blk_status fp8_grouped_block_gemm(const void *x_q, const float *x_scale,
                                                const void *w_q, const float *w_scale,
                                                const int32_t *expert_offsets, int32_t E,
                                                int64_t total_M, int64_t N, int64_t K,
                                                void *y_bf16, void *stream);

/* The whole FP8 linear layer, y = x * W^T from bf16 x: dynamic activation
 * quantization then the block-scaled GEMM ("DeepGEMM fast path"; the
 * quantization "fused ahead of the GEMM").  For M <= 64 (decode) one kernel
 * can do both: the activation codes and scales are formed in registers
 * inside the weight-streaming GEMM and never reach memory.  It is used when
 * no workspaces are given (x_q_ws and x_scale_ws may be NULL for M <= 64;
 * they are then not touched), and with workspaces where it is the faster
 * path: M <= 16 with N * K <= 2^25, or with K <= 8192 and N wide enough for
 * the kernel to pack several 16-column slabs per workgroup; 16 < M <= 32
 * with N * K <= 2^24.
 * Otherwise the two kernels run back to back on `stream` through the
 * caller's workspaces x_q_ws [M,K] and x_scale_ws [M,K/128] (required for
 * M > 64, 16-byte aligned), which then hold the activation codes and
 * scales.  The activation codes and scales are always
 * those of fp8_act_quant_group; y is bit-identical to fp8_act_quant_group
 * followed by fp8_block_gemm wherever that GEMM runs its decode kernel
 * (M <= 32, and 32 < M <= 64 with N < 12288 and K <= 16384: the same K
 * split over the same waves); where it runs a tiled kernel instead
 * (32 < M <= 64 with N >= 12288 or K > 16384, reached by the fused kernel
 * only without workspaces) the fp32 partial sums are added in another
 * order.  It takes no GEMM workspace and so never the K splits of
 * fp8_block_gemm_ws (small grids, stream-K tail, decode with long K);
 * callers that want them run fp8_act_quant_group then fp8_block_gemm_ws.
 *   x_bf16 [M,K], w_q [N,K], w_scale [ceil(N/128),K/128] in; y_bf16 [M,N] out. */
FP8BLK_API fp8blk_status fp8_linear(const void *x_bf16, int64_t M, int64_t N, int64_t K,
                                    const void *w_q, const float *w_scale, void *x_q_ws,
                                    float *x_scale_ws, void *y_bf16, void *stream);

/* Batched (fixed-capacity) expert layout.  "Fine-grained FP8" page,
 * "UE8M0 scale format": the batched_mm expert back-end takes fp32 scales
 * directly.  Reading fixed here: expert e owns a slab of `capacity` rows of
 * which the first counts[e] (clamped to [0, capacity]) hold tokens.
 *   x_q [E*capacity, K], x_scale [E*capacity, K/128]  (i.e. [E, C, ...])
 *   w_q [E,N,K], w_scale [E, ceil(N/128), K/128]
 *   expert_counts: DEVICE int32 [E] (trusted, read on the device)
 *   y_bf16 [E*capacity, N] out; rows past an expert's count are not written. */
FP8BLK_API fp8blk_status fp8_batched_block_gemm(const void *x_q, const float *x_scale,
                                                const void *w_q, const float *w_scale,
                                                const int32_t *expert_counts, int32_t E,
                                                int64_t capacity, int64_t N, int64_t K,
                                                void *y_bf16, void *stream);

/* ------------------------------------------------------------------------
 * Row-wise scales ("fp8r").
 * "BFL (fp8r / nvfp4)" page of the diffusers docs, introduction: one fp32
 * weight scale per row, activations quantized row-wise at run time;
 * "Kernels": a row-scaled fp8 matrix product.  Readings fixed here: the
 * element map of the block scheme with the set = one whole row of K values
 * (s = fl32(amax_row / 448), q = E4M3_RNE(fl32(x / s)), all-zero rows get
 * s = 0); y[m,n] = bf16( x_scale[m] * w_scale[n] * sum_k dec(x_q[m,k])
 * dec(w_q[n,k]) ) with fp32 accumulation.  K must be a multiple of 128 as
 * everywhere else. */

/* Row-wise quantization (weights: R = N output rows; activations: R = M
 * tokens).  in_bf16 [R,K] in; q [R,K] E4M3 codes out; scale [R] fp32 out. */
FP8BLK_API fp8blk_status fp8_rowwise_quant(const void *in_bf16, int64_t R, int64_t K, void *q,
                                           float *scale, void *stream);

/* Row-scaled FP8 GEMM.  x_q [M,K], x_scale [M], w_q [N,K], w_scale [N] in;
 * y_bf16 [M,N] out. */
FP8BLK_API fp8blk_status fp8_rowwise_gemm(const void *x_q, const float *x_scale,
                                          const void *w_q, const float *w_scale,
                                          int64_t M, int64_t N, int64_t K,
                                          void *y_bf16, void *stream);

/* ------------------------------------------------------------------------
 * SwiGLU ahead of the activation quantizer (the quantized input of a
 * mixture-of-experts down projection).  "Fine-grained FP8" page: experts
 * run through grouped back-ends with fp32 scales, and activations are
 * quantized per token per 128-channel group at run time ("DeepGEMM fast
 * path").  The pages do not spell SwiGLU out; readings fixed here:
 *   gate_up_bf16 [M, 2I] in: gate g in columns [0, I), up u in [I, 2I);
 *   h = bf16_RNE(SiLU(g) * u), SiLU(g) = g / (1 + e^-g), evaluated in
 *   binary64 (its bf16 rounding is the exact value's except within ~2^-52
 *   of a rounding midpoint);
 *   x_q [M, I] E4M3 codes and x_scale [M, I/128] fp32 out: exactly
 *   fp8_act_quant_group applied to h (h itself is never written).
 * I must be a positive multiple of 128 and M * I / 128 < 2^31
 * (FP8BLK_ERR_SHAPE).  Every h must be finite (|SiLU(g) * u| below bf16's
 * overflow threshold); otherwise the codes of its group are unspecified. */
FP8BLK_API fp8blk_status fp8_swiglu_act_quant(const void *gate_up_bf16, int64_t M, int64_t I,
                                              void *x_q, float *x_scale, void *stream);

/* The same with power-of-two scales ("UE8M0 scale format"): x_scale [M, I/128]
 * E8M0 bytes (no alignment needed), exactly fp8_act_quant_group_ue8m0
 * applied to h. */
FP8BLK_API fp8blk_status fp8_swiglu_act_quant_ue8m0(const void *gate_up_bf16, int64_t M,
                                                    int64_t I, void *x_q, uint8_t *x_scale,
                                                    void *stream);

/* ------------------------------------------------------------------------
 * Static activation scale.
 * "Fine-grained FP8" page, "DeepGEMM fast path": besides the dynamic scheme
 * the page names static activation quantization (its back-ends keep it on
 * the Triton path).  Readings fixed here: one calibrated fp32 scale s for
 * the whole activation tensor, supplied by the caller in DEVICE memory (one
 * float, 4-byte aligned; it may change between calls without a host sync),
 * with the meaning of the dynamic scales (x ~= dec(q) * s);
 * q = E4M3_RNE(sat(fl32(x / s))), the IEEE quotient saturated to +-448 (the
 * inputs may exceed the calibrated range).  s must be positive and finite;
 * otherwise results are unspecified (the kernels stay in bounds). */

/* Static activation quantization.
 *   x_bf16 [M,K] bf16 in; x_scale DEVICE fp32 [1] in; x_q [M,K] E4M3 out. */
FP8BLK_API fp8blk_status fp8_act_quant_static(const void *x_bf16, int64_t M, int64_t K,
                                              const float *x_scale, void *x_q, void *stream);

/* Block-scaled FP8 GEMM with one static activation scale:
 * y[m,n] = bf16( sum_kb x_scale * w_scale[n/128,kb] * sum_{k in kb}
 *                dec(x_q[m,k]) dec(w_q[n,k]) ), fp32 accumulation.
 *   x_q [M,K], x_scale DEVICE fp32 [1], w_q [N,K], w_scale [ceil(N/128),K/128]
 *   in; y_bf16 [M,N] out. */
FP8BLK_API fp8blk_status fp8_block_gemm_static(const void *x_q, const float *x_scale,
                                               const void *w_q, const float *w_scale,
                                               int64_t M, int64_t N, int64_t K,
                                               void *y_bf16, void *stream);

/* ------------------------------------------------------------------------
 * Power-of-two scales stored as E8M0 bytes.
 * "Fine-grained FP8" page, "UE8M0 scale format": pre-quantized
 * DeepSeek-V4-style checkpoints keep their scales as packed float8_e8m0fnu
 * (scale_fmt = "ue8m0") instead of fp32.  Readings fixed here:
 *   - E8M0 is the OCP MX scale type: byte b encodes 2^(b - 127), 0xFF is NaN,
 *     there is no zero.  One byte per scale, in the same layouts as the fp32
 *     scales above ("packed" = 1 byte instead of 4).
 *   - The scale of a block or group is 2^e, e the smallest integer >= -127
 *     with amax <= 448 * 2^e (rounded up, so no code saturates); the byte is
 *     e + 127 (never 0xFF for finite input; an all-zero set gets 0x00).
 *   - q = E4M3_RNE(x * 2^-e), an exact quotient.
 *   - Activations are quantized with power-of-two scales too, so both GEMM
 *     operands carry E8M0 bytes and the matrix core applies them (each
 *     128-block product enters the fp32 accumulator already scaled).
 * Everything else (shapes, validation, errors, streams) is as above. */

/* Weight quantization with E8M0 block scales.
 *   w_bf16 [N,K] bf16 in; w_q [N,K] E4M3 codes out;
 *   w_scale [ceil(N/128), K/128] E8M0 bytes out (blocks as above). */
FP8BLK_API fp8blk_status fp8_weight_block_quant_ue8m0(const void *w_bf16, int64_t N, int64_t K,
                                                      void *w_q, uint8_t *w_scale,
                                                      void *stream);

/* Dynamic activation quantization with E8M0 group scales.
 *   x_bf16 [M,K] bf16 in; x_q [M,K] E4M3 codes out;
 *   x_scale [M, K/128] E8M0 bytes out (groups as above). */
FP8BLK_API fp8blk_status fp8_act_quant_group_ue8m0(const void *x_bf16, int64_t M, int64_t K,
                                                   void *x_q, uint8_t *x_scale, void *stream);

/* Block-scaled FP8 GEMM with E8M0 scales on both operands, y = x * W^T in
 * bf16: y[m,n] = sum_kb 2^(x_scale[m,kb]-127) * 2^(w_scale[n/128,kb]-127) *
 * sum_{k in kb} dec(x_q[m,k]) dec(w_q[n,k]), fp32 accumulation.
 *   x_q [M,K], x_scale [M,K/128] bytes, w_q [N,K],
 *   w_scale [ceil(N/128),K/128] bytes in; y_bf16 [M,N] out. */
FP8BLK_API fp8blk_status fp8_block_gemm_ue8m0(const void *x_q, const uint8_t *x_scale,
                                              const void *w_q, const uint8_t *w_scale,
                                              int64_t M, int64_t N, int64_t K,
                                              void *y_bf16, void *stream);

/* The E8M0 GEMM with K split over workgroups through a caller workspace,
 * exactly as fp8_block_gemm_ws is to fp8_block_gemm (same operation and
 * passage as fp8_block_gemm_ue8m0; the K ranges hold an even number of K
 * blocks, so shapes with an odd K/128 are never split).  Without a usable
 * workspace the call is fp8_block_gemm_ue8m0, bit for bit. */
FP8BLK_API size_t fp8_block_gemm_ue8m0_workspace_bytes(int64_t M, int64_t N, int64_t K);
FP8BLK_API fp8blk_status fp8_block_gemm_ue8m0_ws(const void *x_q, const uint8_t *x_scale,
                                                 const void *w_q, const uint8_t *w_scale,
                                                 int64_t M, int64_t N, int64_t K,
                                                 void *y_bf16, void *workspace,
                                                 size_t workspace_bytes, void *stream);

/* Grouped variant with E8M0 scales (mixture-of-experts; "UE8M0 scale
 * format": such checkpoints also run the expert matmuls).  Arguments as for
 * fp8_grouped_block_gemm, with x_scale [total_M,K/128] and
 * w_scale [E, ceil(N/128), K/128] as E8M0 bytes. */
FP8BLK_API fp8blk_status fp8_grouped_block_gemm_ue8m0(const void *x_q, const uint8_t *x_scale,
                                                      const void *w_q, const uint8_t *w_scale,
                                                      const int32_t *expert_offsets, int32_t E,
                                                      int64_t total_M, int64_t N, int64_t K,
                                                      void *y_bf16, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
FP8BLK_API const char *fp8blk_status_string(int status);

/* FP8BLK_ABI_VERSION of the built library. */
FP8BLK_API int fp8blk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
