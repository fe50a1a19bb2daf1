/*
 * fp8fg -- fine-grained FP8 (E4M3) quantisation and block-scaled FP8 GEMM
 * for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is caller-owned DEVICE memory unless stated
 * otherwise; the library never allocates, frees or retains a caller buffer,
 * never synchronises the stream and never prints.  Each call validates its
 * arguments on the host, enqueues its kernels on `stream` and returns a
 * status code; nothing throws across the ABI.  A device-side fault (for
 * example a pointer to freed memory) is not detected here and surfaces at the
 * caller's next synchronisation of the stream.  Outputs must not alias inputs.
 *
 * The method (sources, cited by page title and section):
 *  - "DeepSeek-V3 FP8 training notes" (innerforce.co.kr board post),
 *    Figure 7(a) passage: activations are grouped and scaled per 1x128 tile
 *    (one token, 128 channels), weights per 128x128 block (128 output x 128
 *    input channels); each group's largest magnitude is mapped onto the
 *    largest finite FP8 value.  Its accumulation passage: FP8 GEMM partial
 *    sums are carried in FP32, and the dequantisation (multiplying by the
 *    group scales) is folded into that higher-precision accumulation.
 *  - yunhecapital.com report, section 2.2.3: 1x128 group-wise activation and
 *    128x128 block-wise weight quantisation; MMA partials promoted to FP32
 *    registers at a fixed accumulation interval.
 *  - tonho.wtf encyclopedia entry "DeepSeek-V3", section "como funciona":
 *    factors computed online, always E4M3, partials promoted to FP32 every 128
 *    elements.  Section "o que isso custou": gradient operands use 1x128 tiles.
 *
 * Numeric contract of the quantisers (bit-exact, identical on every call):
 *    per group   amax = max|x|,  s = fl32(amax / 448),
 *                inv  = (s == 0) ? 0 : fl32(1 / s),
 *                q    = E4M3_RNE_SATURATE(fl32(x * inv))   (sign of x kept)
 *  where E4M3 is the OCP 8-bit E4M3 ("E4M3FN") encoding: bias 7, largest
 *  finite value 448 (code 0x7E), no infinities, NaN never produced for finite
 *  input.  Inputs must be finite and each group's amax must be 0 or at least
 *  448 * 2^-126; other inputs give unspecified codes (never a fault).
 *
 * Dequantised value of an operand element:  dec(q) * scale of its group.
 * GEMM result:  Y[m,n] = sum_k deqA[m,k] * deqB[n,k]   (Y = A * B^T; both
 * operands K-contiguous, as a linear layer's Y = X * W^T).
 */
#ifndef FP8FG_H
#define FP8FG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8FG_ABI_VERSION 9

/* Status codes returned by every entry point. */
enum {
  FP8FG_OK = 0,
  FP8FG_ERR_INVALID_ARG = 1, /* null pointer, negative size, unknown enum value  */
  FP8FG_ERR_UNSUPPORTED = 2, /* valid but outside this library: K % 128 != 0,
                                N % 128 != 0, an unsupported stride layout,
                                a size that overflows the kernels' indexing     */
  FP8FG_ERR_MISALIGNED = 3,  /* a base pointer or row pitch below the required
                                alignment (documented per entry point)          */
  FP8FG_ERR_HIP = 4          /* the HIP runtime refused a launch               */
};

/* Element types of high-precision inputs/outputs. */
enum { FP8FG_F32 = 0, FP8FG_BF16 = 1 };

/* Scale layout of the GEMM's second operand B [N, K]. */
enum {
  FP8FG_B_BLOCK_128x128 = 0, /* sb[N/128, K/128]: 128x128-quantised weights      */
  FP8FG_B_ROW_1x128 = 1      /* sb[N, K/128]: 1x128 tiles along K (gradient-style
                                operand, e.g. the weight-gradient GEMM)           */
};

/* How the FP8 products of each 128-element K block are summed before the
 * block's partial is scaled and added to the FP32 accumulator. */
enum {
  /* gfx950 FP8 matrix cores: within each run of 8 consecutive K the products
   * are aligned to the largest exponent sum and truncated toward zero 13 bits
   * below it (the hardware counterpart of the limited FP8 accumulation the
   * pages report for H800); runs are summed in FP32.  Full FP8 rate. */
  FP8FG_ACCUM_FP8_MFMA = 0,
  /* FP8 operands widened exactly to fp16 on chip and multiplied on the fp16
   * matrix cores: every product is exact and sums are FP32.  Half rate.  Use
   * when the output is FP32 and FP32-level agreement is required. */
  FP8FG_ACCUM_EXACT = 1,
  /* Power-of-two scales only (as written by the *_pow2 quantisers): the
   * scales enter the matrix-core instruction as E8M0 exponents (the
   * group-scaled MMA on the tonho.wtf page's wish list, "o que isso custou";
   * the microscaling formats of the innerforce notes' Figure 7(a) passage).
   * Products within a K block are summed as in FP8FG_ACCUM_FP8_MFMA, scaled
   * exactly by 2^(ea+eb), and added to the FP32 accumulator inside the same
   * instruction, so there is no separate promotion step.  Requires
   * FP8FG_B_BLOCK_128x128 and N % 256 == 0 (FP8FG_ERR_UNSUPPORTED otherwise).
   * A scale that is not a power of two is read as 2^(its fp32 exponent):
   * unspecified results, never a fault.  Zero scales (all-zero groups) are
   * fine: their codes are zero. */
  FP8FG_ACCUM_SCALED_MFMA = 2
};

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void* fp8fg_stream_t;

/*
 * 1x128 activation quantisation (Figure 7(a) passage of the innerforce notes;
 * yunhecapital section 2.2.3; tonho.wtf "como funciona").
 *
 * x       logical matrix [M, K] of `x_dtype` (FP8FG_F32 or FP8FG_BF16): element
 *         (m, k) is at x + m*stride_m + k*stride_k (strides in elements).
 *         Groups run along K: group (m, g) is x[m, 128g .. 128g+127].
 *         Two layouts are accepted:
 *           stride_k == 1  (row-contiguous; stride_m >= K): the forward case.
 *           stride_m == 1  (column-contiguous; stride_k >= M): x is physically
 *                          [K, M] row-major and is read transposed -- the
 *                          gradient-operand case where tiles run along the
 *                          token axis (tonho.wtf "o que isso custou").
 * q       out, uint8 E4M3 codes [M, K] row-major (always K-contiguous).
 * scales  out, fp32 [M, K/128] row-major.
 * Requires K % 128 == 0.  Row-contiguous: x 16-byte aligned and
 * stride_m * sizeof(elem) % 16 == 0.  Column-contiguous: M % 8 == 0, x 16-byte
 * aligned and stride_k * sizeof(elem) % 16 == 0.  q 16-byte aligned, scales
 * 4-byte aligned.  M == 0 is a no-op.
 */
int fp8_quant_act_1x128(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                        int64_t stride_k, uint8_t* q, float* scales, fp8fg_stream_t stream);

/*
 * The same with power-of-two group scales (for FP8FG_ACCUM_SCALED_MFMA).  The
 * microscaling reading of the innerforce notes' Figure 7(a) passage: per group
 *     s = 2^e, e the smallest integer with amax <= 448 * 2^e  (0 if amax == 0),
 *     q = E4M3_RNE(fl32(x * 2^-e))       (exact scaling; |x * 2^-e| <= 448)
 * so the largest code of a nonzero group lies in [0x76, 0x7E].  Arguments,
 * layouts and requirements as fp8_quant_act_1x128; amax must be 0 or at least
 * 448 * 2^-126.
 */
int fp8_quant_act_1x128_pow2(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                             int64_t stride_k, uint8_t* q, float* scales, fp8fg_stream_t stream);

/*
 * Per-tensor quantisation: ONE scale for the whole tensor, the practice the
 * 1x128 / 128x128 grouping replaces (innerforce notes, Figure 7(a) passage),
 * for measuring what the fine-grained grouping buys.  The rule is the
 * fine-grained one with the group being the whole tensor:
 *     s = fl32(amax_all / 448), inv = s ? fl32(1/s) : 0, q = E4M3_RNE(fl32(x * inv)).
 * The scale is written into every entry of a scale array of the layout the
 * GEMM takes, so the codes and scales feed fp8_block_gemm unchanged.
 *
 * x             [M, K] of `x_dtype`, row-contiguous with row pitch ld >= K.
 * q             out, uint8 E4M3 codes [M, K] row-major.
 * scales        out, fp32, every entry = s:
 *                 scale_layout FP8FG_B_ROW_1x128:    [M, K/128]  (activation / A layout)
 *                 scale_layout FP8FG_B_BLOCK_128x128: [M/128, K/128] (weight / B layout;
 *                                                      requires M % 128 == 0)
 *               The array also serves as the kernels' scratch between their
 *               launches (per-block maxima); its contents are final when the
 *               stream reaches the end of the call.
 * Three kernels are enqueued (block maxima, their maximum, the cast), so x is
 * read twice.  Requires K % 128 == 0; x 16-byte aligned with ld * sizeof(elem)
 * % 16 == 0; q 16-byte aligned; scales 4-byte aligned.  M == 0 is a no-op.
 */
int fp8_quant_per_tensor(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                         float* scales, int scale_layout, fp8fg_stream_t stream);

/*
 * 128x128 weight quantisation (same passages).
 *
 * w       [N, K] of `w_dtype`, row pitch ld_w >= K elements; W is [out, in]:
 *         block (i, j) is rows 128i.. (output channels) x columns 128j.. (input).
 * q       out, uint8 codes [N, K] row-major.
 * scales  out, fp32 [N/128, K/128] row-major.
 * Requires N % 128 == 0 and K % 128 == 0; w 16-byte aligned with
 * ld_w * sizeof(elem) % 16 == 0; q 16-byte aligned.  N == 0 is a no-op.
 */
int fp8_quant_weight_128x128(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                             uint8_t* q, float* scales, fp8fg_stream_t stream);

/* The same with power-of-two block scales (rule as fp8_quant_act_1x128_pow2). */
int fp8_quant_weight_128x128_pow2(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, float* scales, fp8fg_stream_t stream);

/*
 * A layer step's two quantisations in one launch: the 1x128 quantisation of a
 * row-contiguous activation and the 128x128 quantisation of a weight (the
 * passages of fp8_quant_act_1x128 and fp8_quant_weight_128x128).  Every code
 * and scale equals what those two calls write; one launch instead of two saves
 * a kernel ramp and tail (X [4096,7168] + W [7168,7168] bf16: 38 us against
 * 43 us).
 *
 * x, x_dtype, M, K_x   activation [M, K_x], row pitch ld_x >= K_x elements
 *                      (the row-contiguous layout of fp8_quant_act_1x128).
 * q_x, s_x             out, codes [M, K_x] and scales [M, K_x/128].
 * w, w_dtype, N, K_w   weight [N, K_w], row pitch ld_w >= K_w elements.
 * q_w, s_w             out, codes [N, K_w] and scales [N/128, K_w/128].
 * pow2                 0: scales amax/448; 1: power-of-two scales (the rule of
 *                      the *_pow2 quantisers), for both tensors.
 * Requirements of each part as in the separate calls; an empty part (M == 0,
 * N == 0 or a zero K) is skipped and its pointers are not read.  The two parts
 * must not overlap.  If either part is invalid nothing is launched and its
 * status is returned (the activation's first).
 */
int fp8_quant_act_weight(const void* x, int x_dtype, int64_t M, int64_t K_x, int64_t ld_x, uint8_t* q_x,
                         float* s_x, const void* w, int w_dtype, int64_t N, int64_t K_w, int64_t ld_w,
                         uint8_t* q_w, float* s_w, int pow2, fp8fg_stream_t stream);

/*
 * 128x128 weight quantisation that also writes the transposed operand, for the
 * data-gradient GEMM dX = dY * W (the "transposed read" the tonho.wtf
 * "DeepSeek-V3" page lists among its hardware wishes, "o que isso custou").
 * A 128x128 block of W^T is the transpose of a block of W with the same amax,
 * so the 128x128 quantisation of W^T is exactly the transposed codes with the
 * transposed scale grid.  Both come from one read of W.
 *
 * w, N, K, ld_w, q, scales   as fp8_quant_weight_128x128 (same bytes written).
 * q_t       out, uint8 codes [K, N] row-major: q_t[k, n] == q[n, k].
 * scales_t  out, fp32 [K/128, N/128] row-major: scales_t[j, i] == scales[i, j].
 * With these, fp8_block_gemm(q_dy, s_dy, q_t, scales_t, FP8FG_B_BLOCK_128x128,
 * ...) computes dX [M, K] = dY [M, N] * W [N, K], where (q_dy, s_dy) is the
 * 1x128 quantisation of dY along N.
 * Requirements as fp8_quant_weight_128x128, plus q_t 16-byte aligned and
 * scales_t 4-byte aligned; no output may alias another.  N == 0 is a no-op.
 */
int fp8_quant_weight_128x128_dual(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, float* scales, uint8_t* q_t, float* scales_t,
                                  fp8fg_stream_t stream);
/* The same with power-of-two block scales (rule as fp8_quant_act_1x128_pow2),
 * for the data gradient on the scaled MFMA (FP8FG_ACCUM_SCALED_MFMA). */
int fp8_quant_weight_128x128_dual_pow2(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                       uint8_t* q, float* scales, uint8_t* q_t, float* scales_t,
                                       fp8fg_stream_t stream);

/*
 * Block-scaled FP8 GEMM  Y = deq(A) * deq(B)^T  (innerforce accumulation
 * passage; yunhecapital section 2.2.3; tonho.wtf "como funciona").
 * For every 128-element K block kb the FP8 partial P_kb[m,n] is formed on the
 * matrix cores, then promoted:
 *     acc[m,n] += P_kb[m,n] * sa[m,kb] * sb(n,kb)      (FP32)
 * with sb(n,kb) = sb[n/128, kb] (FP8FG_B_BLOCK_128x128) or sb[n, kb]
 * (FP8FG_B_ROW_1x128).  Y is acc rounded to `y_dtype` (bf16: round to nearest
 * even).
 *
 * a   uint8 E4M3 [M, K] row-major;   sa fp32 [M, K/128]
 * b   uint8 E4M3 [N, K] row-major;   sb as above
 * y   out, [M, N] row-major of y_dtype
 * Requires K % 128 == 0 and N % 128 == 0 (M is arbitrary); a, b, y 16-byte
 * aligned; sa, sb 4-byte aligned.  M == 0 is a no-op.
 * FP8FG_F32 output when the output tiles fill the device's compute units at
 * least once (e.g. the weight gradient 7168 x 7168): the tiles of the partial
 * last round are split along K over the compute units that round would leave
 * idle, and the parts add their fp32 sums into y (zeroed by the library on
 * `stream` first) with hardware fp32 atomic adds, which need y in ordinary
 * (coarse-grained) device memory such as hipMalloc or PyTorch returns.  The
 * accuracy is unchanged, but the order of those additions, and so the last
 * bits of those tiles, can vary from run to run.  Smaller problems and bf16
 * outputs are computed in a fixed order.
 * The partials are summed as FP8FG_ACCUM_EXACT for FP8FG_F32 output (so FP32
 * outputs agree with the exact result to FP32 accuracy) and as
 * FP8FG_ACCUM_FP8_MFMA for FP8FG_BF16 output; fp8_block_gemm_accum chooses.
 */
int fp8_block_gemm(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                   int b_scale_mode, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                   fp8fg_stream_t stream);

/*
 * fp8_block_gemm with the summation of the FP8 partials chosen by `accum`
 * (FP8FG_ACCUM_FP8_MFMA, FP8FG_ACCUM_EXACT or FP8FG_ACCUM_SCALED_MFMA; the
 * last requires FP8FG_B_BLOCK_128x128 and N % 256 == 0).  Other arguments,
 * requirements and behaviour as fp8_block_gemm.
 */
int fp8_block_gemm_accum(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                         int b_scale_mode, int accum, void* y, int y_dtype, int64_t M, int64_t N,
                         int64_t K, fp8fg_stream_t stream);

/*
 * The same GEMM with its output cast straight to FP8 for the next layer: the
 * "cast fused" into the producer that the tonho.wtf "DeepSeek-V3" page lists
 * among its hardware wishes ("o que isso custou").  The fp32 accumulators
 * acc[m, n] (as fp8_block_gemm with FP8FG_F32 output returns them, apart from
 * the run-to-run bit differences of its K-split tiles) are
 * quantised 1x128 along N by the rule of fp8_quant_act_1x128 (pow2 == 0) or of
 * fp8_quant_act_1x128_pow2 (pow2 == 1), inside the GEMM's epilogue, so Y never
 * goes to HBM in high precision.
 *
 * a, sa, b, sb, accum, M, N, K   as fp8_block_gemm_accum with FP8FG_B_BLOCK_128x128;
 *           accum FP8FG_ACCUM_FP8_MFMA or FP8FG_ACCUM_SCALED_MFMA
 *           (FP8FG_ACCUM_EXACT: FP8FG_ERR_UNSUPPORTED).
 * q_y     out, uint8 E4M3 codes [M, N] row-major (16-byte aligned).
 * s_y     out, fp32 scales [M, N/128] row-major (4-byte aligned).
 * Requires N % 256 == 0 and K % 128 == 0.  M == 0 is a no-op.
 */
int fp8_block_gemm_quant(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int accum,
                         int pow2, uint8_t* q_y, float* s_y, int64_t M, int64_t N, int64_t K,
                         fp8fg_stream_t stream);

/*
 * Grouped block-scaled FP8 GEMM over mixture-of-experts row segments (the
 * MoE layer with 256 routed experts and top-8 routing, yunhecapital section
 * 2.2.2; no token is dropped, tonho.wtf "como funciona"; activations are
 * dispatched in FP8, innerforce notes).
 *
 * Rows offsets[g] .. offsets[g+1]-1 of A belong to expert g and are
 * multiplied by that expert's weight:  Y[r,:] = deq(A[r,:]) * deq(B[g])^T.
 * a              uint8 E4M3 [M_total, K] row-major;  sa fp32 [M_total, K/128]
 * group_offsets  DEVICE int32 [G+1]: offsets[0] == 0, non-decreasing,
 *                offsets[G] == M_total.  Segments may be empty.  The offsets
 *                stay on the device (no host synchronisation).  Offsets that
 *                break these rules give unspecified rows of Y but never an
 *                access outside a, sa, b, sb or y.
 * b              uint8 E4M3 [G, N, K];  sb fp32 [G, N/128, K/128] (128x128)
 * y              out, [M_total, N] of y_dtype
 * Requires K % 128 == 0, N % 128 == 0; alignment as fp8_block_gemm.
 * M_total == 0 or G == 0 is a no-op.  Partials are summed as in
 * fp8_block_gemm (exact for FP8FG_F32 output, FP8 matrix cores for
 * FP8FG_BF16); fp8_block_grouped_gemm_accum chooses.
 */
int fp8_block_grouped_gemm(const uint8_t* a, const float* sa, const int32_t* group_offsets,
                           int64_t G, const uint8_t* b, const float* sb, void* y, int y_dtype,
                           int64_t M_total, int64_t N, int64_t K, fp8fg_stream_t stream);

/* fp8_block_grouped_gemm with the summation chosen by `accum` (as
 * fp8_block_gemm_accum; FP8FG_ACCUM_SCALED_MFMA requires N % 256 == 0). */
int fp8_block_grouped_gemm_accum(const uint8_t* a, const float* sa, const int32_t* group_offsets,
                                 int64_t G, const uint8_t* b, const float* sb, int accum, void* y,
                                 int y_dtype, int64_t M_total, int64_t N, int64_t K,
                                 fp8fg_stream_t stream);

/*
 * The grouped GEMM reading its rows through an index: FP8 dispatch without a
 * permuted copy of the activations (the innerforce notes dispatch activations
 * in FP8; here the dispatch is the index).  Tokens are quantised once, 1x128,
 * and each routed row is read from its token row where the GEMM needs it.
 *
 * Row r of the grouped problem is token row_index[r]:
 *     Y[r,:] = deq(a_tok[row_index[r], :]) * deq(B[g])^T,  r in segment g.
 * a_tok      uint8 E4M3 [T, K] row-major;  sa_tok fp32 [T, K/128]
 * row_index  DEVICE int32 [M_total], values in [0, T) (values outside are
 *            clamped into it: unspecified rows, never an access outside a_tok)
 * group_offsets, G, b, sb, accum, y, y_dtype, M_total, N, K
 *            as fp8_block_grouped_gemm_accum (y stays in routed-row order).
 * Requires N % 256 == 0, K % 128 == 0, T * K < 2^32 (32-bit row offsets),
 * T >= 1 when M_total > 0; row_index 4-byte aligned; other alignment as
 * fp8_block_gemm.  M_total == 0 or G == 0 is a no-op.
 */
int fp8_block_grouped_gemm_gather(const uint8_t* a_tok, const float* sa_tok, int64_t T,
                                  const int32_t* row_index, const int32_t* group_offsets, int64_t G,
                                  const uint8_t* b, const float* sb, int accum, void* y, int y_dtype,
                                  int64_t M_total, int64_t N, int64_t K, fp8fg_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fp8fg_status_string(int status);

/* FP8FG_ABI_VERSION of the loaded library. */
int fp8fg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8FG_H */
