// C-ABI entry points declared in include/fp8fg.h: argument validation on the
// host, then one kernel launch on the caller's stream.  Validation runs before
// any HIP call, so every error path here is reachable without a GPU.
#include "fp8fg.h"

#include <cstdint>
#include <limits>

#include "launch.h"

namespace {

constexpr int64_t kInt32Max = std::numeric_limits<int32_t>::max();

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_size(int dtype) { return dtype == FP8FG_BF16 ? 2 : 4; }

bool valid_dtype(int d) { return d == FP8FG_F32 || d == FP8FG_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP8FG_OK : FP8FG_ERR_HIP; }

}  // namespace

extern "C" {

int fp8fg_abi_version(void) { return FP8FG_ABI_VERSION; }

const char* fp8fg_status_string(int status) {
  switch (status) {
    case FP8FG_OK: return "ok";
    case FP8FG_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or unknown enum)";
    case FP8FG_ERR_UNSUPPORTED: return "unsupported shape or layout (K and N must be multiples of 128; see fp8fg.h)";
    case FP8FG_ERR_MISALIGNED: return "misaligned pointer or row pitch";
    case FP8FG_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

int quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m, int64_t stride_k, uint8_t* q,
              float* scales, fp8fg_stream_t stream, bool pow2) {
  if (!valid_dtype(x_dtype) || M < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return FP8FG_OK;
  if (K % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!x || !q || !scales) return FP8FG_ERR_INVALID_ARG;
  if (M > kInt32Max || K > kInt32Max || M * (K / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  const int es = elem_size(x_dtype);
  const bool bf16 = x_dtype == FP8FG_BF16;
  if (!aligned(q, 16) || !aligned(scales, 4) || !aligned(x, 16)) return FP8FG_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (stride_k == 1 && stride_m >= K) {
    if ((stride_m * es) % 16 != 0) return FP8FG_ERR_MISALIGNED;
    return hip_status(fp8fg::launch_quant_act_rows(x, bf16, pow2, M, K, stride_m, q, scales, s));
  }
  if (stride_m == 1 && stride_k >= M) {
    if (M % 8 != 0) return FP8FG_ERR_UNSUPPORTED;
    if ((stride_k * es) % 16 != 0) return FP8FG_ERR_MISALIGNED;
    return hip_status(fp8fg::launch_quant_act_cols(x, bf16, pow2, M, K, stride_k, q, scales, s));
  }
  if (stride_m < 0 || stride_k < 0) return FP8FG_ERR_INVALID_ARG;
  return FP8FG_ERR_UNSUPPORTED;
}

// Checks of a 128x128 weight quantisation: FP8FG_OK, an error status, or -1
// when there is nothing to do (N == 0 or K == 0).
int check_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w, const uint8_t* q,
                 const float* scales) {
  if (!valid_dtype(w_dtype) || N < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return -1;
  if (N % 128 != 0 || K % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!w || !q || !scales) return FP8FG_ERR_INVALID_ARG;
  if (ld_w < K) return FP8FG_ERR_INVALID_ARG;
  if ((N / 128) * (K / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 4) || (ld_w * elem_size(w_dtype)) % 16 != 0)
    return FP8FG_ERR_MISALIGNED;
  return FP8FG_OK;
}

// Checks of a 1x128 quantisation of a row-contiguous activation (ld_x >= K):
// FP8FG_OK, an error status, or -1 when there is nothing to do.
int check_act_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ld_x, const uint8_t* q,
                   const float* scales) {
  if (!valid_dtype(x_dtype) || M < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return -1;
  if (K % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!x || !q || !scales) return FP8FG_ERR_INVALID_ARG;
  if (ld_x < K) return FP8FG_ERR_INVALID_ARG;
  if (M > kInt32Max || K > kInt32Max || M * (K / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(scales, 4) || !aligned(x, 16) || (ld_x * elem_size(x_dtype)) % 16 != 0)
    return FP8FG_ERR_MISALIGNED;
  return FP8FG_OK;
}

int quant_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w, uint8_t* q, float* scales,
                 fp8fg_stream_t stream, bool pow2) {
  const int c = check_weight(w, w_dtype, N, K, ld_w, q, scales);
  if (c < 0) return FP8FG_OK;
  if (c != FP8FG_OK) return c;
  return hip_status(fp8fg::launch_quant_weight(w, w_dtype == FP8FG_BF16, pow2, N, K, ld_w, q, scales,
                                               static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fp8_quant_act_1x128(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                        int64_t stride_k, uint8_t* q, float* scales, fp8fg_stream_t stream) {
  return quant_act(x, x_dtype, M, K, stride_m, stride_k, q, scales, stream, false);
}

int fp8_quant_act_1x128_pow2(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                             int64_t stride_k, uint8_t* q, float* scales, fp8fg_stream_t stream) {
  return quant_act(x, x_dtype, M, K, stride_m, stride_k, q, scales, stream, true);
}

int fp8_quant_weight_128x128(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                             uint8_t* q, float* scales, fp8fg_stream_t stream) {
  return quant_weight(w, w_dtype, N, K, ld_w, q, scales, stream, false);
}

int fp8_quant_weight_128x128_pow2(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, float* scales, fp8fg_stream_t stream) {
  return quant_weight(w, w_dtype, N, K, ld_w, q, scales, stream, true);
}

int fp8_quant_act_weight(const void* x, int x_dtype, int64_t M, int64_t K_x, int64_t ld_x, uint8_t* q_x,
                         float* s_x, const void* w, int w_dtype, int64_t N, int64_t K_w, int64_t ld_w,
                         uint8_t* q_w, float* s_w, int pow2, fp8fg_stream_t stream) {
  if (pow2 != 0 && pow2 != 1) return FP8FG_ERR_INVALID_ARG;
  const int cx = check_act_rows(x, x_dtype, M, K_x, ld_x, q_x, s_x);
  const int cw = check_weight(w, w_dtype, N, K_w, ld_w, q_w, s_w);
  if (cx > 0) return cx;
  if (cw > 0) return cw;
  if (cx < 0 && cw < 0) return FP8FG_OK;
  // an empty part launches no workgroups
  if (cx < 0) M = 0;
  if (cw < 0) N = 0;
  return hip_status(fp8fg::launch_quant_act_weight(x, x_dtype == FP8FG_BF16, M, K_x, ld_x, q_x, s_x, w,
                                                   w_dtype == FP8FG_BF16, N, K_w, ld_w, q_w, s_w, pow2 == 1,
                                                   static_cast<hipStream_t>(stream)));
}

int fp8_quant_per_tensor(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                         float* scales, int scale_layout, fp8fg_stream_t stream) {
  if (!valid_dtype(x_dtype) || M < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (scale_layout != FP8FG_B_ROW_1x128 && scale_layout != FP8FG_B_BLOCK_128x128) return FP8FG_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return FP8FG_OK;
  if (K % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (scale_layout == FP8FG_B_BLOCK_128x128 && M % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!x || !q || !scales) return FP8FG_ERR_INVALID_ARG;
  if (ld < K) return FP8FG_ERR_INVALID_ARG;
  if (M > kInt32Max || K > kInt32Max || M * (K / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4) || (ld * elem_size(x_dtype)) % 16 != 0)
    return FP8FG_ERR_MISALIGNED;
  const int64_t n_scales = (scale_layout == FP8FG_B_ROW_1x128 ? M : M / 128) * (K / 128);
  return hip_status(fp8fg::launch_quant_per_tensor(x, x_dtype == FP8FG_BF16, M, K, ld, q, scales, n_scales,
                                                   static_cast<hipStream_t>(stream)));
}

namespace {

int quant_weight_dual(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w, uint8_t* q, float* scales,
                      uint8_t* q_t, float* scales_t, bool pow2, fp8fg_stream_t stream) {
  if (!valid_dtype(w_dtype) || N < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return FP8FG_OK;
  if (N % 128 != 0 || K % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!w || !q || !scales || !q_t || !scales_t) return FP8FG_ERR_INVALID_ARG;
  if (ld_w < K) return FP8FG_ERR_INVALID_ARG;
  if ((N / 128) * (K / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(q_t, 16) || !aligned(scales, 4) || !aligned(scales_t, 4) ||
      (ld_w * elem_size(w_dtype)) % 16 != 0)
    return FP8FG_ERR_MISALIGNED;
  return hip_status(fp8fg::launch_quant_weight_dual(w, w_dtype == FP8FG_BF16, pow2, N, K, ld_w, q, scales, q_t,
                                                    scales_t, static_cast<hipStream_t>(stream)));
}

}  // namespace

int fp8_quant_weight_128x128_dual(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, float* scales, uint8_t* q_t, float* scales_t,
                                  fp8fg_stream_t stream) {
  return quant_weight_dual(w, w_dtype, N, K, ld_w, q, scales, q_t, scales_t, false, stream);
}

int fp8_quant_weight_128x128_dual_pow2(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ld_w,
                                       uint8_t* q, float* scales, uint8_t* q_t, float* scales_t,
                                       fp8fg_stream_t stream) {
  return quant_weight_dual(w, w_dtype, N, K, ld_w, q, scales, q_t, scales_t, true, stream);
}

namespace {

int check_gemm_common(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                      int accum, const void* y, int y_dtype, int64_t M, int64_t N, int64_t K) {
  if (!valid_dtype(y_dtype) || M < 0 || N < 0 || K < 0) return FP8FG_ERR_INVALID_ARG;
  if (accum != FP8FG_ACCUM_FP8_MFMA && accum != FP8FG_ACCUM_EXACT && accum != FP8FG_ACCUM_SCALED_MFMA)
    return FP8FG_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return -1;  // nothing to do
  if (K == 0 || K % 128 != 0 || N % 128 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (!a || !sa || !b || !sb || !y) return FP8FG_ERR_INVALID_ARG;
  if (M > kInt32Max || N > kInt32Max || K > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(y, 16) || !aligned(sa, 4) || !aligned(sb, 4))
    return FP8FG_ERR_MISALIGNED;
  return FP8FG_OK;
}

// Accumulation of the entry points without an `accum` argument: FP32 outputs
// take exact products (the FP32 agreement they are held to), bf16 outputs the
// full-rate FP8 matrix cores.
int default_accum(int y_dtype) { return y_dtype == FP8FG_F32 ? FP8FG_ACCUM_EXACT : FP8FG_ACCUM_FP8_MFMA; }

fp8fg::GemmArgs gemm_args(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, void* y,
                          const int32_t* offsets, int64_t M, int64_t N, int64_t K, int64_t G, bool row_scales,
                          int accum, int y_dtype) {
  fp8fg::GemmArgs g{};
  g.a = a; g.sa = sa; g.b = b; g.sb = sb; g.y = y; g.offsets = offsets;
  g.M = M; g.N = N; g.K = K; g.G = G;
  g.row_scales = row_scales;
  g.exact = accum == FP8FG_ACCUM_EXACT;
  g.scaled = accum == FP8FG_ACCUM_SCALED_MFMA;
  g.y_bf16 = y_dtype == FP8FG_BF16;
  return g;
}

}  // namespace

int fp8_block_gemm_accum(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                         int b_scale_mode, int accum, void* y, int y_dtype, int64_t M, int64_t N,
                         int64_t K, fp8fg_stream_t stream) {
  if (b_scale_mode != FP8FG_B_BLOCK_128x128 && b_scale_mode != FP8FG_B_ROW_1x128)
    return FP8FG_ERR_INVALID_ARG;
  const int c = check_gemm_common(a, sa, b, sb, accum, y, y_dtype, M, N, K);
  if (c < 0) return FP8FG_OK;
  if (c != FP8FG_OK) return c;
  // launch grid: ceil(M/128) * (N/128) blocks
  if (((M + 127) / 128) * (N / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  const fp8fg::GemmArgs g = gemm_args(a, sa, b, sb, y, nullptr, M, N, K, 1, b_scale_mode == FP8FG_B_ROW_1x128,
                                      accum, y_dtype);
  if (g.scaled && (g.row_scales || !fp8fg::fp8_block_kernel_applies(g))) return FP8FG_ERR_UNSUPPORTED;
  return hip_status(fp8fg::launch_block_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8_block_gemm(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                   int b_scale_mode, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                   fp8fg_stream_t stream) {
  return fp8_block_gemm_accum(a, sa, b, sb, b_scale_mode, default_accum(y_dtype), y, y_dtype, M, N, K, stream);
}

int fp8_block_gemm_quant(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int accum,
                         int pow2, uint8_t* q_y, float* s_y, int64_t M, int64_t N, int64_t K,
                         fp8fg_stream_t stream) {
  if (accum == FP8FG_ACCUM_EXACT || (pow2 != 0 && pow2 != 1)) return accum == FP8FG_ACCUM_EXACT
                                                                        ? FP8FG_ERR_UNSUPPORTED
                                                                        : FP8FG_ERR_INVALID_ARG;
  const int c = check_gemm_common(a, sa, b, sb, accum, q_y, FP8FG_BF16, M, N, K);
  if (c < 0) return FP8FG_OK;
  if (c != FP8FG_OK) return c;
  if (!s_y) return FP8FG_ERR_INVALID_ARG;
  if (!aligned(s_y, 4)) return FP8FG_ERR_MISALIGNED;
  if (N % 256 != 0) return FP8FG_ERR_UNSUPPORTED;
  if (((M + 127) / 128) * (N / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  fp8fg::GemmArgs g = gemm_args(a, sa, b, sb, q_y, nullptr, M, N, K, 1, false, accum, FP8FG_BF16);
  g.y_scales = s_y;
  if (!fp8fg::fp8_block_kernel_applies(g)) return FP8FG_ERR_UNSUPPORTED;
  return hip_status(fp8fg::launch_fp8_block_gemm_quant(g, pow2 == 1, static_cast<hipStream_t>(stream)));
}

int fp8_block_grouped_gemm(const uint8_t* a, const float* sa, const int32_t* group_offsets,
                           int64_t G, const uint8_t* b, const float* sb, void* y, int y_dtype,
                           int64_t M_total, int64_t N, int64_t K, fp8fg_stream_t stream) {
  return fp8_block_grouped_gemm_accum(a, sa, group_offsets, G, b, sb, default_accum(y_dtype), y, y_dtype, M_total,
                                      N, K, stream);
}

int fp8_block_grouped_gemm_accum(const uint8_t* a, const float* sa, const int32_t* group_offsets,
                                 int64_t G, const uint8_t* b, const float* sb, int accum, void* y,
                                 int y_dtype, int64_t M_total, int64_t N, int64_t K,
                                 fp8fg_stream_t stream) {
  if (G < 0) return FP8FG_ERR_INVALID_ARG;
  const int c = check_gemm_common(a, sa, b, sb, accum, y, y_dtype, M_total, N, K);
  if (c < 0 || G == 0) return c > 0 ? c : FP8FG_OK;
  if (c != FP8FG_OK) return c;
  if (!group_offsets) return FP8FG_ERR_INVALID_ARG;
  if (!aligned(group_offsets, 4)) return FP8FG_ERR_MISALIGNED;
  if (G > kInt32Max || (M_total / 128 + G) * (N / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  const fp8fg::GemmArgs g = gemm_args(a, sa, b, sb, y, group_offsets, M_total, N, K, G, false, accum, y_dtype);
  if (g.scaled && !fp8fg::fp8_block_kernel_applies(g)) return FP8FG_ERR_UNSUPPORTED;
  return hip_status(fp8fg::launch_grouped_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8_block_grouped_gemm_gather(const uint8_t* a_tok, const float* sa_tok, int64_t T, const int32_t* row_index,
                                  const int32_t* group_offsets, int64_t G, const uint8_t* b, const float* sb,
                                  int accum, void* y, int y_dtype, int64_t M_total, int64_t N, int64_t K,
                                  fp8fg_stream_t stream) {
  if (G < 0 || T < 0) return FP8FG_ERR_INVALID_ARG;
  const int c = check_gemm_common(a_tok, sa_tok, b, sb, accum, y, y_dtype, M_total, N, K);
  if (c < 0 || G == 0) return c > 0 ? c : FP8FG_OK;
  if (c != FP8FG_OK) return c;
  if (T == 0 || !group_offsets || !row_index) return FP8FG_ERR_INVALID_ARG;
  if (!aligned(group_offsets, 4) || !aligned(row_index, 4)) return FP8FG_ERR_MISALIGNED;
  if (G > kInt32Max || (M_total / 128 + G) * (N / 128) > kInt32Max) return FP8FG_ERR_UNSUPPORTED;
  if (T > kInt32Max || T * K >= (int64_t(1) << 32)) return FP8FG_ERR_UNSUPPORTED;  // 32-bit row offsets
  fp8fg::GemmArgs g = gemm_args(a_tok, sa_tok, b, sb, y, group_offsets, M_total, N, K, G, false, accum, y_dtype);
  g.row_index = row_index;
  g.T = T;
  if (!fp8fg::fp8_block_kernel_applies(g)) return FP8FG_ERR_UNSUPPORTED;  // N % 256 != 0
  return hip_status(fp8fg::launch_grouped_gemm_gather(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
