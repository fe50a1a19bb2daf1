// Block-scaled FP8 GEMM on gfx950 matrix cores, dense and grouped.
//
// Y[m,n] = sum_kb  P_kb[m,n] * sa[m,kb] * sb(n,kb),  P_kb = sum_{k in kb} a[m,k] b[n,k]
// (FP8 partial per 128-element K block, promoted to FP32 and scaled at the block
// boundary: accumulation passage of the innerforce DeepSeek-V3 notes;
// yunhecapital report section 2.2.3; tonho.wtf "DeepSeek-V3", "como funciona").
//
// Mapping to the hardware:
//  * One 128-wide K block is one LDS stage and one scale step.  A and B tiles
//    (128 bytes of K per row) are staged global -> registers -> LDS, double
//    buffered, with 16-byte chunks XOR-swizzled by (row & 7) so that the
//    fragment reads of 16 consecutive rows spread over all banks.
//  * The matrix-core operands are swapped (MFMA "A" = rows of B, MFMA "B" = rows
//    of A), so each lane's four results of a 16x16 sub-tile share one m and four
//    consecutive n.  With 128x128 weight blocks the promotion factor
//    sa[m,kb]*sb[n/128,kb] is then one value per lane and sub-tile column:
//    one FMA per output per K block on the vector ALU, overlapping the MFMAs.
//  * FP8 accumulation: v_mfma_f32_16x16x128_f8f6f4 forms the whole 128-K partial
//    in one instruction (zero C input).  Exact accumulation: the FP8 fragments
//    are widened to fp16 (exact) and summed with four v_mfma_f32_16x16x32_f16.
//  * The grouped kernel maps each workgroup to (expert, m-tile, n-tile) from the
//    device-resident segment offsets; rows past a segment's end are loaded from
//    a clamped in-segment row and never stored.
#include "launch.h"

namespace fp8fg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;  // K bytes per stage == scale block

struct Params {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* y;
  const int32_t* offsets;
  int64_t M, N, K, G;
  int KB;  // K / 128
  int NT;  // N / BN
};

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
// Two fp32 values rounded to nearest-even bf16 and packed (low half a): one
// v_cvt_pk_bf16_f32 on gfx950, bit-identical to the integer rounding
// ((u + 0x7FFF + lsb) >> 16) for finite values.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ v8h widen8(uint32_t lo, uint32_t hi) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(lo), 1.0f, false);
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(lo), 1.0f, true);
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(hi), 1.0f, false);
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(hi), 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// 128-K partial of one 16x16 sub-tile: MFMA A = rows of the weight-side operand.
template <bool EXACT>
__device__ __forceinline__ v4f partial(const v8i& fa, const v8i& fb) {
  v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (!EXACT) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, z, 0, 0, 0, 0, 0, 0);
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      v8h ha = widen8(static_cast<uint32_t>(fa[2 * p]), static_cast<uint32_t>(fa[2 * p + 1]));
      v8h hb = widen8(static_cast<uint32_t>(fb[2 * p]), static_cast<uint32_t>(fb[2 * p + 1]));
      z = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, z, 0, 0, 0);
    }
    return z;
  }
}

// Read a 16-row x 128-byte fragment in the 16x16x128 operand layout: lane l
// takes row (l % 16) and bytes 32*(l/16) .. +31, i.e. chunks 2j and 2j+1.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row0, int lane) {
  const int row = row0 + (lane & 15);
  const int j = lane >> 4;
  const int sw = row & 7;
  const u32x4* r = reinterpret_cast<const u32x4*>(tile + row * BK);
  u32x4 c0 = r[(2 * j) ^ sw];
  u32x4 c1 = r[(2 * j + 1) ^ sw];
  v8i f;
  f[0] = c0[0]; f[1] = c0[1]; f[2] = c0[2]; f[3] = c0[3];
  f[4] = c1[0]; f[5] = c1[1]; f[6] = c1[2]; f[7] = c1[3];
  return f;
}

template <int BM, int BN, int WM, int WN, bool EXACT, bool ROWS, bool BF16OUT, bool GROUPED>
__global__ void __launch_bounds__(WM* WN * 64) gemm_kernel(Params p) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int SM = TM / 16, SN = TN / 16;  // 16x16 sub-tiles per wave
  constexpr int A_CH = BM * 8 / NTHR;        // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 8 / NTHR;
  constexpr int SB_PER = ROWS ? BN : BN / 128;
  static_assert(BM * 8 % NTHR == 0 && BN * 8 % NTHR == 0, "tile/threads");
  static_assert(BN % 128 == 0 || ROWS, "block scales need 128-aligned n tiles");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * BK];
  __shared__ float lds_sa[2][BM];
  __shared__ float lds_sb[2][SB_PER];
  __shared__ int tile_info[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  // ---- which output tile
  int64_t row_lo, row_hi;  // rows [row_lo, row_hi) of A / Y handled here (row_hi - row_lo <= BM)
  const uint8_t* bmat = p.b;
  const float* bscale = p.sb;
  const int nt = blockIdx.x % p.NT;
  const int mt = blockIdx.x / p.NT;
  if constexpr (!GROUPED) {
    row_lo = static_cast<int64_t>(mt) * BM;
    row_hi = row_lo + BM < p.M ? row_lo + BM : p.M;
  } else {
    // Wave 0 scans the per-expert tile counts to find the expert owning m-tile mt.
    if (wave == 0) {
      int running = 0;
      int found = -1, f_lo = 0, f_hi = 0;
      const int64_t Mt = p.M;
      for (int64_t base = 0; base < p.G; base += 64) {
        const int64_t g = base + lane;
        int64_t lo = 0, hi = 0;
        if (g < p.G) {
          lo = p.offsets[g];
          hi = p.offsets[g + 1];
          lo = lo < 0 ? 0 : (lo > Mt ? Mt : lo);
          hi = hi < lo ? lo : (hi > Mt ? Mt : hi);
        }
        const int cnt = static_cast<int>((hi - lo + BM - 1) / BM);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          int o = __shfl_up(incl, d);
          if (lane >= d) incl += o;
        }
        const int excl = running + incl - cnt;
        const bool mine = (cnt > 0) && (mt >= excl) && (mt < excl + cnt);
        const unsigned long long who = __ballot(mine);
        if (who) {
          const int src = __ffsll(who) - 1;
          const int64_t my_lo = lo + static_cast<int64_t>(mt - excl) * BM;
          const int64_t my_hi = my_lo + BM < hi ? my_lo + BM : hi;
          found = __shfl(static_cast<int>(g), src);
          f_lo = __shfl(static_cast<int>(my_lo), src);
          f_hi = __shfl(static_cast<int>(my_hi), src);
          break;
        }
        running += __shfl(incl, 63);
        if (running > mt) break;
      }
      if (lane == 0) {
        tile_info[0] = found;
        tile_info[1] = f_lo;
        tile_info[2] = f_hi;
      }
    }
    __syncthreads();
    const int g = tile_info[0];
    if (g < 0) return;  // whole block leaves together
    row_lo = tile_info[1];
    row_hi = tile_info[2];
    bmat += static_cast<int64_t>(g) * p.N * p.K;
    bscale += static_cast<int64_t>(g) * (p.N / 128) * p.KB;
  }
  const int64_t n0 = static_cast<int64_t>(nt) * BN;

  // ---- global -> register staging
  u32x4 ra[A_CH], rb[B_CH];
  float rsa = 0.0f, rsb = 0.0f;
  auto load_stage = [&](int kb) {
    const int64_t kof = static_cast<int64_t>(kb) * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NTHR;
      const int r = c >> 3, ch = c & 7;
      int64_t row = row_lo + r;
      row = row < row_hi ? row : row_hi - 1;
      ra[i] = *reinterpret_cast<const u32x4*>(p.a + row * p.K + kof + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NTHR;
      const int r = c >> 3, ch = c & 7;
      rb[i] = *reinterpret_cast<const u32x4*>(bmat + (n0 + r) * p.K + kof + ch * 16);
    }
    if (tid < BM) {
      int64_t row = row_lo + tid;
      row = row < row_hi ? row : row_hi - 1;
      rsa = p.sa[row * p.KB + kb];
    }
    if (tid < SB_PER) {
      if constexpr (ROWS)
        rsb = bscale[(n0 + tid) * p.KB + kb];
      else
        rsb = bscale[(n0 / 128 + tid) * p.KB + kb];
    }
  };
  auto store_stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NTHR;
      const int r = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(&lds_a[st][r * BK + ((ch ^ (r & 7)) * 16)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NTHR;
      const int r = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(&lds_b[st][r * BK + ((ch ^ (r & 7)) * 16)]) = rb[i];
    }
    if (tid < BM) lds_sa[st][tid] = rsa;
    if (tid < SB_PER) lds_sb[st][tid] = rsb;
  };

  v4f acc[SN][SM];
#pragma unroll
  for (int i = 0; i < SN; ++i)
#pragma unroll
    for (int j = 0; j < SM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int KB = p.KB;
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < KB) load_stage(kb + 1);

    const uint8_t* ta = lds_a[st];
    const uint8_t* tb = lds_b[st];
    v8i fm[SM];
    float fsa[SM];
#pragma unroll
    for (int j = 0; j < SM; ++j) {
      fm[j] = read_frag(ta, wm * TM + j * 16, lane);
      fsa[j] = lds_sa[st][wm * TM + j * 16 + (lane & 15)];
    }
    if constexpr (!ROWS) {
      const float sbv = lds_sb[st][(wn * TN) / 128];
#pragma unroll
      for (int j = 0; j < SM; ++j) fsa[j] *= sbv;
    }
#pragma unroll
    for (int i = 0; i < SN; ++i) {
      const v8i fn = read_frag(tb, wn * TN + i * 16, lane);
      float fsb[4];
      if constexpr (ROWS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) fsb[r] = lds_sb[st][wn * TN + i * 16 + 4 * (lane >> 4) + r];
      }
#pragma unroll
      for (int j = 0; j < SM; ++j) {
        const v4f P = partial<EXACT>(fn, fm[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (ROWS)
            acc[i][j][r] = fmaf(P[r], fsa[j] * fsb[r], acc[i][j][r]);
          else
            acc[i][j][r] = fmaf(P[r], fsa[j], acc[i][j][r]);
        }
      }
    }

    if (kb + 1 < KB) store_stage(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds Y[m][n .. n+3] for m = column, n = 4 consecutive rows
#pragma unroll
  for (int j = 0; j < SM; ++j) {
    const int64_t m = row_lo + wm * TM + j * 16 + (lane & 15);
    if (m >= row_hi) continue;
#pragma unroll
    for (int i = 0; i < SN; ++i) {
      const int64_t n = n0 + wn * TN + i * 16 + 4 * (lane >> 4);
      if constexpr (BF16OUT) {
        u32x2 o;
        o[0] = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
        o[1] = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.y) + m * p.N + n) = o;
      } else {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.y) + m * p.N + n) = acc[i][j];
      }
    }
  }
}

constexpr int kBM = 128, kBN = 128, kWM = 2, kWN = 2;

template <bool EXACT, bool ROWS, bool BF16OUT, bool GROUPED>
hipError_t launch_t(const Params& p, unsigned blocks, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<kBM, kBN, kWM, kWN, EXACT, ROWS, BF16OUT, GROUPED>), dim3(blocks),
                     dim3(kWM * kWN * 64), 0, s, p);
  return hipGetLastError();
}

template <bool GROUPED>
hipError_t dispatch(const GemmArgs& g, unsigned blocks, hipStream_t s) {
  Params p{g.a, g.sa, g.b, g.sb, g.y, g.offsets, g.M, g.N, g.K, g.G,
           static_cast<int>(g.K / 128), static_cast<int>(g.N / kBN)};
  const int key = (g.exact ? 4 : 0) | (g.row_scales ? 2 : 0) | (g.y_bf16 ? 1 : 0);
  switch (key) {
    case 0: return launch_t<false, false, false, GROUPED>(p, blocks, s);
    case 1: return launch_t<false, false, true, GROUPED>(p, blocks, s);
    case 2: return launch_t<false, true, false, GROUPED>(p, blocks, s);
    case 3: return launch_t<false, true, true, GROUPED>(p, blocks, s);
    case 4: return launch_t<true, false, false, GROUPED>(p, blocks, s);
    case 5: return launch_t<true, false, true, GROUPED>(p, blocks, s);
    case 6: return launch_t<true, true, false, GROUPED>(p, blocks, s);
    default: return launch_t<true, true, true, GROUPED>(p, blocks, s);
  }
}

}  // namespace

hipError_t launch_block_gemm(const GemmArgs& g, hipStream_t s) {
  if (fp8_block_kernel_applies(g)) return launch_fp8_block_gemm(g, false, s);
  const int64_t mt = (g.M + kBM - 1) / kBM;
  const int64_t nt = g.N / kBN;
  return dispatch<false>(g, static_cast<unsigned>(mt * nt), s);
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s) {
  if (fp8_block_kernel_applies(g)) return launch_fp8_block_gemm(g, true, s);
  // Upper bound on m-tiles: sum_g ceil(rows_g / BM) <= M_total / BM + G.
  const int64_t mt = g.M / kBM + g.G;
  const int64_t nt = g.N / kBN;
  return dispatch<true>(g, static_cast<unsigned>(mt * nt), s);
}

}  // namespace fp8fg
