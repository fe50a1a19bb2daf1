// Throughput kernel for the block-scaled FP8 GEMM with 128x128 weight scales
// and FP8 matrix-core accumulation (the dense projection and the MoE grouped
// GEMM).  Same contract as gemm.hip:
//   Y[m,n] = sum_kb P_kb[m,n] * sa[m,kb] * sb[n/128,kb],  P_kb = FP8 partial of
//   K block kb, promoted to FP32 and scaled at the block boundary
// (innerforce DeepSeek-V3 notes, accumulation passage; yunhecapital report
// section 2.2.3; tonho.wtf "DeepSeek-V3", "como funciona").
//
// Layout on gfx950:
//  * 256 x 256 output tile per 512-thread workgroup: 8 wavefronts (2 per SIMD)
//    arranged 2 (n) x 4 (m), each 128 (n) x 64 (m) = 8 x 4 sub-tiles of 16 x 16.
//    At this size the L2 -> CU traffic (64 KB per 16.8 MFLOP) stays within what
//    the L2 delivers to 256 CUs while the matrix cores run at full rate.
//  * One 128-wide K block per LDS stage (64 KB), two stages: the loads of block
//    kb+1 are issued while block kb is multiplied.
//  * Tiles move global -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//    issued through inline assembly together with the waits and barriers: the
//    compiler cannot tell that an LDS read does not overlap the DMA writes still
//    in flight, and would otherwise drain every load before every read.
//    Each DMA instruction fills 8 rows x 128 bytes; every lane reads 16 bytes of
//    a full 128-byte row segment (the access pattern the L2 serves fastest).
//    In LDS the 16-byte chunks of row r are permuted by XOR with (r & 7), and a
//    lane of a fragment read takes logical chunks j and j+4 (j = lane / 16) of
//    row lane % 16: measured bank-conflict free for ds_read_b128 on gfx950.
//  * The per-block scales are staged the same way (global_load_lds_dword).
//  * v_mfma_f32_16x16x128_f8f6f4 forms each sub-tile's 128-K partial; the
//    promotion acc += P * sa[m,kb] * sb[nb,kb] is one VALU FMA per output, the
//    factor being one value per lane and sub-tile column because the MFMA
//    operands are swapped (MFMA "A" = weight rows).  The partials are double
//    buffered so the FMAs of one sub-tile run under the MFMAs of the next.
//  * Tiles are numbered so that each XCD (workgroup id mod 8) works on one
//    contiguous band of the tile grid, keeping its operand panels in its L2.
#include "launch.h"

namespace fp8fg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256;
constexpr int NTHREADS = 512;
constexpr int TM = 64, TN = 128;  // wavefront tile (m, n)
constexpr int SM = TM / 16, SN = TN / 16;
constexpr int TILE_A = BM * 128;          // 32 KB
constexpr int TILE_B = BN * 128;          // 32 KB
constexpr int STAGE = TILE_A + TILE_B;    // 64 KB
constexpr int GROUP_M = 4;                // m-tiles per band in the dense tile order

struct FParams {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* y;
  const int32_t* offsets;
  int64_t M, N, K, G;
  int KB;  // K / 128
  int MT;  // m-tiles (dense: ceil(M/BM); grouped: upper bound M/BM + G)
  int NT;  // N / BN
};

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Fragment of tile rows row0 .. row0+15 in the 16x16x128 operand layout: lane
// l takes row row0 + l%16, logical 16-byte chunks j and j+4 (j = l/16), stored
// at physical chunk positions (c ^ (row & 7)).
__device__ __forceinline__ v8i frag(const uint8_t* tile, int row0, int lane) {
  const int row = row0 + (lane & 15);
  const int j = lane >> 4;
  const u32x4* p = reinterpret_cast<const u32x4*>(tile + row * 128);
  const u32x4 c0 = p[j ^ (row & 7)];
  const u32x4 c1 = p[(j + 4) ^ (row & 7)];
  v8i f;
  f[0] = c0[0]; f[1] = c0[1]; f[2] = c0[2]; f[3] = c0[3];
  f[4] = c1[0]; f[5] = c1[1]; f[6] = c1[2]; f[7] = c1[3];
  return f;
}

// LDS DMA: 64 lanes x 16 bytes (or 4 bytes) from per-lane global addresses to
// 1 KB (256 B) of LDS starting at the wave-uniform byte address `lds`.
// M0 is written here and nowhere else in the kernel (no other instruction of
// this kernel reads M0), so it needs no saving.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory");
}
// Wait until all of this wavefront's loads and LDS reads have completed, then
// synchronise the workgroup: after it, the next K block is resident and the
// stage read in this iteration may be refilled by any wavefront.
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <bool BF16OUT, bool GROUPED>
__global__ void __launch_bounds__(NTHREADS, 1) gemm_fp8_block_kernel(FParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float s_sa[2][BM];
  __shared__ __attribute__((aligned(16))) float s_sb[2][64];
  __shared__ int tile_info[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;  // 4 wavefronts along m, 2 along n

  // ---- tile selection
  const int T = p.MT * p.NT;
  const int bid = blockIdx.x;
  const int t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  int mt, nt;
  if constexpr (!GROUPED) {
    const int band = t / (GROUP_M * p.NT);
    const int first = band * GROUP_M;
    const int gsz = (p.MT - first) < GROUP_M ? (p.MT - first) : GROUP_M;
    const int r = t - band * GROUP_M * p.NT;
    mt = first + r % gsz;
    nt = r / gsz;
  } else {
    nt = t / p.MT;  // m-tiles of one n-panel are consecutive: the expert's B panel stays in L2
    mt = t % p.MT;
  }

  int64_t row_lo, row_hi;
  const uint8_t* bmat = p.b;
  const float* bscale = p.sb;
  if constexpr (!GROUPED) {
    row_lo = static_cast<int64_t>(mt) * BM;
    row_hi = row_lo + BM < p.M ? row_lo + BM : p.M;
  } else {
    if (wave == 0) {
      int running = 0, found = -1, f_lo = 0, f_hi = 0;
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
          const int o = __shfl_up(incl, d);
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
    if (g < 0) return;  // whole workgroup
    row_lo = tile_info[1];
    row_hi = tile_info[2];
    bmat += static_cast<int64_t>(g) * p.N * p.K;
    bscale += static_cast<int64_t>(g) * (p.N / 128) * p.KB;
  }
  const int64_t n0 = static_cast<int64_t>(nt) * BN;

  // ---- per-lane source addresses (rows fixed for the whole K loop).
  // Wavefront w fills rows [32w, 32w+32) of both tiles, 8 rows per DMA: lane L
  // writes physical chunk L%8 of row 8i + L/8, i.e. logical chunk (L%8)^(L/8).
  // Waves 0-3 also load the A scales of 64 rows each, wave 4 the two weight-block
  // scales (lane 0: block n0/128, other lanes: block n0/128 + 1).
  const int lrow = lane >> 3;
  const int lchunk = ((lane & 7) ^ lrow) * 16;
  const uint8_t* ga[4];
  const uint8_t* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + lrow;
    int64_t row = row_lo + r;
    row = row < row_hi ? row : row_hi - 1;
    ga[i] = p.a + row * p.K + lchunk;
    gb[i] = bmat + (n0 + r) * p.K + lchunk;
  }
  const float* gs = nullptr;
  if (wave < 4) {
    int64_t row = row_lo + wave * 64 + lane;
    row = row < row_hi ? row : row_hi - 1;
    gs = p.sa + row * p.KB;
  } else if (wave == 4) {
    gs = bscale + (n0 / 128 + (lane < 1 ? 0 : 1)) * p.KB;
  }
  // wave-uniform LDS destinations (readfirstlane tells the compiler they are scalar)
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_ta = lds_addr(tiles) + uwave * 32 * 128;
  const uint32_t lds_tb = lds_ta + TILE_A;
  const uint32_t lds_s0 = uwave < 4 ? lds_addr(&s_sa[0][uwave * 64]) : lds_addr(&s_sb[0][0]);
  const uint32_t lds_s_step = uwave < 4 ? BM * 4 : 64 * 4;

  auto issue = [&](int kb, int st) {
    const int64_t kof = static_cast<int64_t>(kb) * 128;
    const uint32_t so = static_cast<uint32_t>(st) * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(ga[i] + kof, lds_ta + so + i * 1024);
      dma16(gb[i] + kof, lds_tb + so + i * 1024);
    }
    if (uwave <= 4) dma4(gs + kb, lds_s0 + static_cast<uint32_t>(st) * lds_s_step);
  };

  v4f acc[SN][SM];
#pragma unroll
  for (int i = 0; i < SN; ++i)
#pragma unroll
    for (int j = 0; j < SM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int KB = p.KB;
  issue(0, 0);
  wait_barrier();

  int st = 0;  // stage holding block kb
  for (int kb = 0; kb < KB; ++kb) {
    // Block kb+1 into the other stage (consumed in the previous iteration).  On
    // the last iteration the free stage is refilled with block KB-1, which is
    // not read again: the loop body stays branch-free.
    issue(kb + 1 < KB ? kb + 1 : KB - 1, st ^ 1);

    const uint8_t* tA = tiles + st * STAGE;
    const uint8_t* tB = tA + TILE_A;
    const float sbv = s_sb[st][wn];
    v8i fm[SM];
    float f[SM];
#pragma unroll
    for (int j = 0; j < SM; ++j) {
      fm[j] = frag(tA, wm * TM + j * 16, lane);
      f[j] = s_sa[st][wm * TM + j * 16 + (lane & 15)] * sbv;
    }
    // Software pipeline over the n sub-tiles: the fragment of sub-tile i+1 is
    // read from LDS while the MFMAs of sub-tile i run, and the promotion FMAs of
    // sub-tile i-1 (double-buffered partials) fill the VALU under them.
    v4f P[2][SM];
    v8i fn = frag(tB, wn * TN, lane);
#pragma unroll
    for (int i = 0; i < SN; ++i) {
      v8i fn_next;
      if (i + 1 < SN) fn_next = frag(tB, wn * TN + (i + 1) * 16, lane);
#pragma unroll
      for (int j = 0; j < SM; ++j) {
        const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
        P[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fn, fm[j], z, 0, 0, 0, 0, 0, 0);
      }
      if (i > 0) {
#pragma unroll
        for (int j = 0; j < SM; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = fmaf(P[(i - 1) & 1][j][r], f[j], acc[i - 1][j][r]);
      }
      if (i + 1 < SN) fn = fn_next;
      // Issue order for this step: the next fragment's two LDS reads, then
      // four times (one MFMA, four VALU FMAs of the previous sub-tile).
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int j = 0; j < SM; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < SM; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[SN - 1][j][r] = fmaf(P[(SN - 1) & 1][j][r], f[j], acc[SN - 1][j][r]);

    wait_barrier();  // block kb+1 resident; stage st free for refilling
    st ^= 1;
  }

  // ---- epilogue: lane holds Y[m][n .. n+3], m = sub-tile column, n = 4 consecutive rows
#pragma unroll
  for (int j = 0; j < SM; ++j) {
    const int64_t m = row_lo + wm * TM + j * 16 + (lane & 15);
    if (m >= row_hi) continue;
#pragma unroll
    for (int i = 0; i < SN; ++i) {
      const int64_t n = n0 + wn * TN + i * 16 + 4 * (lane >> 4);
      if constexpr (BF16OUT) {
        u32x2 o;
        o[0] = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
        o[1] = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.y) + m * p.N + n) = o;
      } else {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.y) + m * p.N + n) = acc[i][j];
      }
    }
  }
}

template <bool BF16OUT, bool GROUPED>
hipError_t launch_fp8(const GemmArgs& g, int MT, hipStream_t s) {
  FParams p{g.a, g.sa, g.b, g.sb, g.y, g.offsets, g.M, g.N, g.K, g.G,
            static_cast<int>(g.K / 128), MT, static_cast<int>(g.N / BN)};
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(MT) * p.NT);
  hipLaunchKernelGGL((gemm_fp8_block_kernel<BF16OUT, GROUPED>), dim3(blocks), dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool fp8_block_kernel_applies(const GemmArgs& g) {
  return !g.exact && !g.row_scales && g.N % BN == 0;
}

hipError_t launch_fp8_block_gemm(const GemmArgs& g, bool grouped, hipStream_t s) {
  const int64_t MT = grouped ? g.M / BM + g.G : (g.M + BM - 1) / BM;
  if (grouped)
    return g.y_bf16 ? launch_fp8<true, true>(g, static_cast<int>(MT), s)
                    : launch_fp8<false, true>(g, static_cast<int>(MT), s);
  return g.y_bf16 ? launch_fp8<true, false>(g, static_cast<int>(MT), s)
                  : launch_fp8<false, false>(g, static_cast<int>(MT), s);
}

}  // namespace fp8fg
