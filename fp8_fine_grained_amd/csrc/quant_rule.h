// The per-group quantisation rule, shared by the quantisers (quant.hip) and the
// GEMM epilogue that writes its output already quantised (gemm_fp8.hip).
// Per group (innerforce DeepSeek-V3 notes, Figure 7(a) passage; tonho.wtf
// "DeepSeek-V3", "como funciona"):
//     amax = max|x|,  s = fl32(amax/448),  inv = s ? fl32(1/s) : 0,
//     q = E4M3 RNE cast of fl32(x*inv), sign kept;
// or, with power-of-two scales, s = 2^e for the smallest e with
// amax <= 448 * 2^e and inv = 2^-e (details in quant.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp8fg {

constexpr float kE4M3Max = 448.0f;

template <bool POW2 = false>
__device__ __forceinline__ void group_scale(float amax, float& s, float& inv) {
  if constexpr (!POW2) {
    s = amax / kE4M3Max;
    inv = (s == 0.0f) ? 0.0f : 1.0f / s;
  } else {
    const uint32_t b = __float_as_uint(amax);
    int eb = static_cast<int>(b >> 23) - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);  // biased exponent of s
    eb = eb < 1 ? 1 : eb;  // amax below 448 * 2^-126 (outside the contract): the smallest normal scale
    s = amax == 0.0f ? 0.0f : __uint_as_float(static_cast<uint32_t>(eb) << 23);
    inv = amax == 0.0f ? 0.0f : __uint_as_float(static_cast<uint32_t>(254 - eb) << 23);
  }
}

// Four fp32 values -> four E4M3 bytes (little-endian order a, b, c, d).
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return static_cast<uint32_t>(v);
}

}  // namespace fp8fg
