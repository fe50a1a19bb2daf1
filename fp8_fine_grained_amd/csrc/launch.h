// Internal launcher interface between the C-ABI layer (capi.cpp) and the
// HIP kernels.  Arguments reaching these functions have been validated.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp8fg {

// pow2: power-of-two (E8M0) group scales instead of amax/448.
// 1x128 quantisation, row-contiguous input (stride_k == 1).
hipError_t launch_quant_act_rows(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, int64_t ld,
                                 uint8_t* q, float* scales, hipStream_t s);
// 1x128 quantisation along K of a column-contiguous input (stride_m == 1):
// x is physically [K, ld] row-major, element (m, k) at k*ld + m.
hipError_t launch_quant_act_cols(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, int64_t ld,
                                 uint8_t* q, float* scales, hipStream_t s);
// One scale for the whole row-contiguous [M, K] tensor, written into all
// n_scales entries of `scales` (M * K/128 or (M/128) * (K/128) of them).
hipError_t launch_quant_per_tensor(const void* x, bool bf16, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                                   float* scales, int64_t n_scales, hipStream_t s);
// 128x128 quantisation.
hipError_t launch_quant_weight(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, int64_t ld,
                               uint8_t* q, float* scales, hipStream_t s);
// 128x128 quantisation of w and 1x128 quantisation of the row-contiguous x in one
// launch (either part may be empty: M == 0 or N == 0).
hipError_t launch_quant_act_weight(const void* x, bool x_bf16, int64_t M, int64_t K_x, int64_t ld_x, uint8_t* q_x,
                                   float* s_x, const void* w, bool w_bf16, int64_t N, int64_t K_w, int64_t ld_w,
                                   uint8_t* q_w, float* s_w, bool pow2, hipStream_t s);
// 128x128 quantisation writing q [N,K] and the transposed q_t [K,N] (+ scales, scales_t).
hipError_t launch_quant_weight_dual(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, int64_t ld,
                                    uint8_t* q, float* scales, uint8_t* qt, float* scales_t, hipStream_t s);

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* y;
  const int32_t* offsets;  // grouped only
  int64_t M, N, K, G;
  bool row_scales;  // B scales per row (1x128) instead of per 128x128 block
  bool exact;       // exact products (fp16 matrix cores) instead of FP8 MFMA
  bool scaled;      // power-of-two scales applied by the matrix cores (E8M0), FP32 accumulation in the MFMA
  bool y_bf16;
  const int32_t* row_index = nullptr;  // grouped with gather: row r of A is a[row_index[r]]
  int64_t T = 0;                       // rows of a (and sa) when gathering
  float* y_scales = nullptr;           // quantised output: scales [M, N/128] (y = codes [M, N])
};
hipError_t launch_block_gemm(const GemmArgs& g, hipStream_t s);
hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s);
// Grouped GEMM gathering A rows by index (requires fp8_block_kernel_applies).
hipError_t launch_grouped_gemm_gather(const GemmArgs& g, hipStream_t s);

// 256x256-tile FP8-accumulation kernel for 128x128 weight scales (gemm_fp8.hip).
bool fp8_block_kernel_applies(const GemmArgs& g);
hipError_t launch_fp8_block_gemm(const GemmArgs& g, bool grouped, hipStream_t s);
// Dense GEMM writing its output as 1x128-quantised E4M3 codes (g.y) and scales
// (g.y_scales); requires N % 256 == 0, block-scaled B, FP8 or scaled accumulation.
hipError_t launch_fp8_block_gemm_quant(const GemmArgs& g, bool pow2, hipStream_t s);

}  // namespace fp8fg
