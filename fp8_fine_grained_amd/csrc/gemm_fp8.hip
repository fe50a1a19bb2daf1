// Throughput kernel for the block-scaled FP8 GEMM with 128x128 weight scales
// and FP8 matrix-core accumulation (the dense projection and the MoE grouped
// GEMM).  Same contract as gemm.hip:
//   Y[m,n] = sum_kb P_kb[m,n] * sa[m,kb] * sb[n/128,kb],  P_kb = FP8 partial of
//   K block kb, promoted to FP32 and scaled at the block boundary
// (innerforce DeepSeek-V3 notes, accumulation passage; yunhecapital report
// section 2.2.3; tonho.wtf "DeepSeek-V3", "como funciona").
//
// Layout on gfx950:
//  * 512-thread workgroups (8 wavefronts, 2 per SIMD; the template also takes 4,
//    one per SIMD), each wavefront owning a (TN x TM) block of 16 x 16
//    sub-tiles.  Tile shapes:
//      dense   256 (m) x 256 (n), wavefronts 4 (m) x 2 (n) of 64 x 128, 2 stages;
//      dense, power-of-two scales: 256 x 256, wavefronts 2 x 2 of 128 x 128;
//      grouped 128 (m) x 256 (n), wavefronts 2 (m) x 4 (n) of 64 x 64, 3 stages
//    (128-row tiles waste less of the last tile of each ~256-row expert segment).
//    With 256 x 256 the L2 -> CU traffic is 64 KB per 16.8 MFLOP.
//  * One 128-wide K block per LDS stage; the loads of block kb+STAGES-1 are in
//    flight while block kb is multiplied.  They are issued over the first six
//    of the eight sub-tile steps (four for the fp32-scale dense tiles; 128 x 256
//    tiles: the first three of four when grouped, else the first two), one or two
//    DMAs per step between MFMAs: early enough to land before the end of the
//    iteration, spread out because each DMA costs the issuing wavefront and the
//    LDS both per instruction and per byte.  The power-of-two tiles, the
//    grouped FP8 tiles and the fp32-scale dense tiles with block scales place
//    each of a step's DMAs right after one of its MFMAs, in an order fixed by
//    scheduling barriers.
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
//  * Dense 256 x 256 tiles also touch K block kb+3 while multiplying block kb
//    (one dword per 128-byte line, each line once per XCD), so operands that
//    only HBM holds (just written by the quantisers) reach L2 before the DMAs
//    of block kb+2 ask for them; without it the GEMM runs ~12% slower right
//    after the quantisers than back to back.
//  * v_mfma_f32_16x16x128_f8f6f4 forms each sub-tile's 128-K partial; the
//    promotion acc += P * sa[m,kb] * sb[nb,kb] is one VALU FMA per output, the
//    factor being one value per lane and sub-tile column because the MFMA
//    operands are swapped (MFMA "A" = weight rows).  The partials are double
//    buffered so the FMAs of one sub-tile run under the MFMAs of the next.  The
//    barrier of each K block comes right after its last LDS read: the last
//    sub-tile's MFMAs and FMAs run after it, while the next block's fragments
//    are being read (FP8 and scaled tiles: its n fragment and scales first,
//    then one m fragment after each MFMA).
//  * Dense tiles are numbered so that each XCD (workgroup id mod 8) works on one
//    contiguous band of the tile grid, keeping its operand panels in its L2;
//    grouped tiles are in expert-major order, so one XCD works through one
//    expert's tiles at a time.
//  * Grouped tiles multiply only the 16-row sub-tiles that hold rows of the
//    expert's segment: the K loop is compiled for 1 .. SM row sub-tiles and a
//    wavefront runs the copy for its live rows, chosen once per tile.
#include <atomic>
#include <type_traits>

#include "launch.h"
#include "quant_rule.h"

namespace fp8fg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int GROUP_M = 4;     // m-tiles per band in the dense tile order

struct FParams {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* y;
  const int32_t* offsets;
  const int32_t* rows;  // gather: row r of the grouped problem is row rows[r] of a / sa
  int64_t M, N, K, G, T;
  int KB;  // K / 128
  int MT;  // m-tiles (dense: ceil(M/BM); grouped: upper bound M/BM + G)
  int NT;  // N / BN
  float* ys;  // quantised output: 1x128 scales [M, N/128] (y holds the E4M3 codes [M, N])
  // Dense fp32 outputs: tiles 0 .. T_full-1 run whole; each later tile (those
  // of a partial last round of the CUs) is split into `split` K ranges run by
  // separate workgroups, which add their fp32 results into the zeroed output.
  int T_full;
  int split;
};

// Dense tile order: bands of GROUP_M m-tiles, n-tile major inside a band, so the
// tiles an XCD runs together share their A and B panels.
__device__ __forceinline__ void dense_tile_coords(int t, int MT, int NT, int& mt, int& nt) {
  const int band = t / (GROUP_M * NT);
  const int first = band * GROUP_M;
  const int gsz = (MT - first) < GROUP_M ? (MT - first) : GROUP_M;
  const int r = t - band * GROUP_M * NT;
  mt = first + r % gsz;
  nt = r / gsz;
}

// Two fp32 values rounded to nearest-even bf16 and packed (low half a): one
// v_cvt_pk_bf16_f32 on gfx950, bit-identical to the integer rounding
// ((u + 0x7FFF + lsb) >> 16) it replaces; on the power-of-two dense GEMM and
// the gathering MoE GEMM 1.2% and 0.7% faster (their epilogues convert 256 and
// 64 outputs per lane per tile).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
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

// Exact widening of 8 E4M3 codes (two dwords) to fp16: every E4M3 value,
// subnormals included, is an fp16 value.
__device__ __forceinline__ v8h widen8(uint32_t lo, uint32_t hi) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(lo), 1.0f, false);
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(lo), 1.0f, true);
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(hi), 1.0f, false);
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(hi), 1.0f, true);
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// A fragment widened for four 16x16x32 fp16 MFMAs: part q holds the lane's
// bytes 8q .. 8q+7 of its 32, so across the four lane groups part q covers 32
// of the 128 K values, and A and B are split the same way.
struct WideFrag {
  v8h q[4];
};
__device__ __forceinline__ WideFrag widen(const v8i& f) {
  WideFrag w;
#pragma unroll
  for (int q = 0; q < 4; ++q) w.q[q] = widen8(static_cast<uint32_t>(f[2 * q]), static_cast<uint32_t>(f[2 * q + 1]));
  return w;
}

// LDS DMA: 64 lanes x 16 bytes (or 4 bytes) to 1 KB (256 B) of LDS starting
// at the wave-uniform byte address `lds`.  The tile form takes a wave-uniform
// base (SGPR pair) plus a fixed 32-bit per-lane offset, so advancing to the
// next K block is a scalar add and the instruction reads one address VGPR.
// The LDS address is taken from M0, which the DMA may read only one wait state
// after a scalar ALU write (gfx9 hazard; the compiler places the same s_nop 0
// for its own LDS-DMA builtin, but cannot see inside this asm).  M0 is a
// reserved register to the compiler, so it cannot be listed as clobbered; the
// compiled kernels name M0 nowhere but in these helpers and have no other
// instruction that reads it (both checked on the gfx950 assembly by the
// library's static device-code test), so writing it here disturbs nothing.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory");
}
// The same with only the lanes of `mask` active.  The instruction is always
// issued (no branch around it), so every wavefront's count of outstanding
// loads per stage stays the same whatever the mask.
__device__ __forceinline__ void dma16_masked(const uint8_t* base, uint32_t voff, uint32_t lds, uint64_t mask) {
  // (the mask is wave-uniform; readfirstlane keeps it in scalar registers.  Its
  // int results are widened as uint32: a sign-extended low word would switch on
  // lanes 32-63 whenever lane 31 is live.)
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(mask >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(mask)));
  mask = (static_cast<uint64_t>(hi) << 32) | lo;
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %4\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base), "s"(mask)
      : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory");
}
// Wait until at most N of this wavefront's loads are outstanding (those of the
// newer blocks) and all of its LDS reads have completed, then
// synchronise the workgroup: after it, the next K block is resident and the
// stage read in this iteration may be refilled by any wavefront.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// BM x BN output tile (m x n), WM x WN wavefronts, STAGES K blocks in LDS.
// EXACT: operands widened to fp16 and multiplied by fp16 MFMAs (every product and
// every in-instruction sum exact); ROWS: one weight-side scale per row n and
// K block instead of one per 128 x 128 block.
// GATHER (grouped only): A rows and their scales are read through p.rows.
// SCALED: power-of-two scales applied by the matrix cores (E8M0 operands of the
// scaled MFMA), which also accumulate: no separate promotion step.
// QOUT: the output leaves quantised, 1x128 along N, by the quantisers' rule
// applied to the fp32 accumulators (1: scale amax/448, 2: power-of-two scale).
template <int BM, int BN, int WM, int WN, int STAGES, bool EXACT, bool ROWS, bool BF16OUT, bool GROUPED,
          bool GATHER = false, bool SCALED = false, int QOUT = 0>
__global__ void __launch_bounds__(WM * WN * 64, 1) gemm_fp8_block_kernel(FParams p) {
  constexpr int NW = WM * WN;  // wavefronts: 8 (2 per SIMD) or 4 (1 per SIMD)
  static_assert(NW == 8 || NW == 4, "8 or 4 wavefronts");
  constexpr int TM = BM / WM, TN = BN / WN;  // wavefront tile (m, n)
  constexpr int SM = TM / 16, SN = TN / 16;
  // BALIGN: tiles start on weight-block boundaries and a wavefront's n range lies
  // in one weight block, so one block factor serves the wavefront; otherwise
  // (224-wide tiles) each 16-wide sub-tile takes the factor of its own block.
  constexpr bool BALIGN = BN % 128 == 0 && (TN % 128 == 0 || 128 % TN == 0);
  static_assert(ROWS || BALIGN || (BN % 32 == 0 && !GROUPED), "unaligned weight tiles: dense, 32-row multiples");
  constexpr int TILE_A = BM * 128;
  constexpr int TILE_B = BN * 128;
  constexpr int STAGE = TILE_A + TILE_B;
  // 8-row DMAs per wavefront per stage.  B row groups are dealt out in
  // contiguous runs when they divide evenly over the 8 wavefronts, else
  // round-robin (group w + 8d for DMA d), the missing last ones masked off.
  constexpr int B_GROUPS = BN / 8;
  constexpr bool B_RR = B_GROUPS % NW != 0;
  static_assert(BM % (8 * NW) == 0, "whole A DMAs per wavefront");
  constexpr int A_DMA = BM / 8 / NW, B_DMA = (B_GROUPS + NW - 1) / NW;
  constexpr int SA_WAVES = BM / 64;                  // wavefronts loading the A scales (64 rows each)
  constexpr int SB_WAVES = ROWS ? BN / 64 : 1;       // and the B scales (64 rows, or all blocks)
  // With four wavefronts and 256 rows every wavefront loads A scales and
  // wavefront 0 also the weight-block scales (two scale DMAs; two stages only,
  // where every wait drains all loads, so the uneven count does not matter).
  constexpr bool SB_EXTRA = SA_WAVES + SB_WAVES > NW;
  static_assert(!SB_EXTRA || (SA_WAVES == NW && !ROWS && STAGES == 2), "one scale DMA per wavefront");
  constexpr int SB_LEN = ROWS ? BN : 64;
  constexpr int NB = BALIGN ? BN / 128 : BN / 128 + 2;  // weight blocks a tile can touch (block mode)
  // loads per wavefront per stage: tiles + one scale (or filler) DMA
  constexpr int LOADS = A_DMA + B_DMA + 1;
  constexpr int WAIT_N = (STAGES - 2) * LOADS;
  static_assert(STAGES >= 2, "at least double buffering");
  static_assert(!(ROWS && GROUPED), "grouped weights carry block scales");
  static_assert(!GATHER || GROUPED, "gathering is a grouped-GEMM mode");
  static_assert(!SCALED || (!EXACT && !ROWS), "the scaled mode takes FP8 products and 128x128 weight scales");
  static_assert(QOUT == 0 || (TN == 128 && BALIGN && !GROUPED), "a wavefront's row of the tile is one 1x128 group");
  // bf16 epilogue: each wavefront stages its TM x TN result (rows of TN*2 bytes
  // padded by 16) in its own slice of the tile buffer.
  constexpr int EPI_PITCH = TN * 2 + 16;
  constexpr int EPI_BYTES = NW * TM * EPI_PITCH;
  constexpr int TILES_BYTES = STAGES * STAGE > EPI_BYTES ? STAGES * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[TILES_BYTES];
  __shared__ __attribute__((aligned(16))) float s_sa[STAGES][BM];
  __shared__ __attribute__((aligned(16))) float s_sb[STAGES][SB_LEN];
  __shared__ __attribute__((aligned(16))) float s_filler[64];  // landing slot of the filler DMAs, never read
  __shared__ int tile_info[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Wavefronts w and w + 4 share a SIMD.  Grouped tiles put the m-halves (or
  // quarters) of the tile on different wavefronts of each SIMD pair, so that a
  // tile holding only a few rows of an expert segment, whose wavefronts past
  // the segment end skip their matrix work, still spreads the remaining
  // MFMAs over the SIMDs.
  const int wm = GROUPED ? wave / WN : wave % WM, wn = GROUPED ? wave % WN : wave / WM;

  // ---- tile selection
  const int T = p.MT * p.NT;
  const int bid = blockIdx.x;
  int t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  // K range of this workgroup (in 128-blocks) and whether it adds into the
  // output: the K-split parts of the tiles past T_full (dense fp32 only) come
  // after the whole tiles in the grid, and the parts of one tile run on
  // consecutive workgroups (so on different XCDs).
  int kb_begin = 0, kb_count = p.KB;
  bool add_out = false;
  if constexpr (!GROUPED && !BF16OUT && QOUT == 0) {
    if (p.split > 1) {
      if (bid < p.T_full) {
        t = (p.T_full % 8 == 0) ? (bid % 8) * (p.T_full / 8) + bid / 8 : bid;
      } else {
        const int u = bid - p.T_full;
        const int part = u % p.split;
        t = p.T_full + u / p.split;
        kb_begin = static_cast<int>(static_cast<int64_t>(part) * p.KB / p.split);
        kb_count = static_cast<int>(static_cast<int64_t>(part + 1) * p.KB / p.split) - kb_begin;
        add_out = true;
      }
    }
  }
  int mt, nt;
  if constexpr (GROUPED) {
    // The grid covers an upper bound of the m-tiles; the live ones are counted
    // here (from the device offsets) and dealt out in equal XCD bands, so that
    // the workgroups left over, which exit at once, are spread over all XCDs
    // instead of filling the last bands.
    if (wave == 0) {
      int total = 0;
      for (int64_t base = 0; base < p.G; base += 64) {
        const int64_t g = base + lane;
        int cnt = 0;
        if (g < p.G) {
          int64_t lo = p.offsets[g], hi = p.offsets[g + 1];
          lo = lo < 0 ? 0 : (lo > p.M ? p.M : lo);
          hi = hi < lo ? lo : (hi > p.M ? p.M : hi);
          cnt = static_cast<int>((hi - lo + BM - 1) / BM);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d);
        total += cnt;
      }
      if (lane == 0) tile_info[0] = total;
    }
    __syncthreads();
    const int live = tile_info[0] * p.NT;  // <= T
    if (T % 8 == 0) {
      const int band = (live + 7) / 8;
      t = bid / 8 < band ? (bid % 8) * band + bid / 8 : T;  // T: no tile
    }
    __syncthreads();  // tile_info is rewritten below
  }
  if constexpr (!GROUPED) {
    dense_tile_coords(t, p.MT, p.NT, mt, nt);
  } else {
    // Expert-major order: the m-tiles of all experts are concatenated and tile
    // t belongs to m-tile t / NT's expert; that expert's mt_g x NT tiles are
    // consecutive in t (n-tile major), so one XCD works through one expert at
    // a time and its weight panel and token rows are each fetched about once.
    mt = t / p.NT;
    nt = 0;
  }

  int64_t row_lo, row_hi;
  const uint8_t* bmat = p.b;
  const float* bscale = p.sb;
  if constexpr (!GROUPED) {
    row_lo = static_cast<int64_t>(mt) * BM;
    row_hi = row_lo + BM < p.M ? row_lo + BM : p.M;
  } else {
    if (wave == 0) {
      int running = 0, found = -1, f_lo = 0, f_hi = 0, f_nt = 0;
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
          const int g_excl = __shfl(excl, src);
          const int g_cnt = __shfl(cnt, src);
          const int g_lo = __shfl(static_cast<int>(lo), src);
          const int g_hi = __shfl(static_cast<int>(hi), src);
          const int local = t - g_excl * p.NT;
          f_nt = local / g_cnt;
          f_lo = g_lo + (local % g_cnt) * BM;
          f_hi = f_lo + BM < g_hi ? f_lo + BM : g_hi;
          found = __shfl(static_cast<int>(g), src);
          break;
        }
        running += __shfl(incl, 63);
        if (running > mt) break;
      }
      if (lane == 0) {
        tile_info[0] = found;
        tile_info[1] = f_lo;
        tile_info[2] = f_hi;
        tile_info[3] = f_nt;
      }
    }
    __syncthreads();
    const int g = tile_info[0];
    if (g < 0) return;  // whole workgroup
    row_lo = tile_info[1];
    row_hi = tile_info[2];
    nt = tile_info[3];
    bmat += static_cast<int64_t>(g) * p.N * p.K;
    bscale += static_cast<int64_t>(g) * (p.N / 128) * p.KB;
  }
  const int64_t n0 = static_cast<int64_t>(nt) * BN;

  // ---- per-lane source addresses (rows fixed for the whole K loop).
  // Wavefront w fills A rows [w*BM/8, (w+1)*BM/8) and B rows [w*BN/8, ...),
  // 8 rows per DMA: lane L writes physical chunk L%8 of row 8i + L/8, i.e.
  // logical chunk (L%8)^(L/8).  Wavefronts 0..SA_WAVES-1 also load the A scales
  // of 64 rows each, wavefront SA_WAVES the weight-block scales (lane i: block
  // n0/128 + min(i, BN/128-1)); the others load a filler value into a scratch
  // slot, so every wavefront issues exactly LOADS loads per stage.
  const int lrow = lane >> 3;
  const int lchunk = ((lane & 7) ^ lrow) * 16;
  // Source row of A (and of its scales) for tile row `row` (in [row_lo, row_hi)).
  auto a_row = [&](int64_t row) -> int64_t {
    if constexpr (GATHER) {
      int64_t t = p.rows[row];
      return t < 0 ? 0 : (t >= p.T ? p.T - 1 : t);
    } else {
      return row;
    }
  };
  // Byte offsets within the tile's row panels (below 256 * K < 2^32), or from
  // the start of A when gathering (below T * K < 2^32).
  // Contiguous operands: every DMA of a wavefront uses the same lane offset
  // (row lrow, chunk lchunk); the wavefront's row block and the DMA's 8-row step
  // are folded into the wave-uniform base.  Gathered rows keep one offset per DMA.
  const int uw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* a_base = uniform_ptr(GATHER ? p.a : p.a + (row_lo + uw * (BM / NW)) * p.K);
  const uint8_t* b_base = uniform_ptr(bmat + (n0 + uw * (B_RR ? 8 : BN / NW)) * p.K);
  const uint32_t voff = static_cast<uint32_t>(lrow * p.K + lchunk);
  uint32_t va[GATHER ? A_DMA : 1];
  uint64_t a_live[A_DMA];  // lanes whose tile row lies inside the segment (or the matrix)
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const int r = wave * (BM / NW) + i * 8 + lrow;
    int64_t row = row_lo + r;
    a_live[i] = __ballot(row < row_hi);
    row = row < row_hi ? row : row_hi - 1;
    if constexpr (GATHER) va[i] = static_cast<uint32_t>(a_row(row) * p.K + lchunk);
  }
  const float* gs;
  if (wave < SA_WAVES) {
    int64_t row = row_lo + wave * 64 + lane;
    row = row < row_hi ? row : row_hi - 1;
    gs = p.sa + a_row(row) * p.KB;
  } else if constexpr (ROWS) {
    int w = wave - SA_WAVES;
    w = w < SB_WAVES ? w : 0;  // filler wavefronts re-read the first weight rows' scales
    gs = bscale + (n0 + w * 64 + lane) * p.KB;
  } else {
    int64_t blk = n0 / 128 + (lane < NB - 1 ? lane : NB - 1);
    blk = blk < p.N / 128 ? blk : p.N / 128 - 1;
    gs = bscale + blk * p.KB;
  }
  // wave-uniform LDS destinations (readfirstlane tells the compiler they are scalar)
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_ta = lds_addr(tiles) + uwave * (BM / NW) * 128;
  const uint32_t lds_tb = lds_addr(tiles) + TILE_A + uwave * (B_RR ? 8 : BN / NW) * 128;
  const bool b_scale_wave = uwave >= SA_WAVES && uwave < SA_WAVES + SB_WAVES;
  const uint32_t lds_s0 = uwave < SA_WAVES ? lds_addr(&s_sa[0][uwave * 64])
                          : (b_scale_wave ? lds_addr(&s_sb[0][(uwave - SA_WAVES) * 64]) : lds_addr(s_filler));
  const uint32_t lds_s_step = uwave < SA_WAVES ? BM * 4 : (b_scale_wave ? SB_LEN * 4 : 0);
  const float* gsb = nullptr;  // weight-block scales of the extra scale DMA
  if constexpr (SB_EXTRA) {
    int64_t blk = n0 / 128 + (lane < NB - 1 ? lane : NB - 1);
    blk = blk < p.N / 128 ? blk : p.N / 128 - 1;
    gsb = bscale + blk * p.KB;
  }

  // L2 prefetch (256 x 256 dense tiles): in iteration kb every wavefront touches
  // one dword of K block kb + PF_DIST in 96 / NW rows, so the lines are on their way
  // from HBM two iterations before the DMAs ask for them (the DMAs' own lead is
  // one iteration, which covers the latency of the last-level cache but not that
  // of HBM, e.g. right after the quantisers have written the operands).  The
  // tiles that run at the same time on one XCD share their panels (with the
  // band order: 8 n-tiles per A panel, 4 m-tiles per B panel), so each tile
  // touches one slice, 32 A rows and 64 B rows, and each line is requested
  // about once per XCD.  The loads land in the LDS filler slot, never read.
  constexpr int PF_DIST = 3;
  constexpr int PF = (GROUPED || BM != 256) ? 0 : PF_DIST;
  const uint8_t* pf_ptr = nullptr;
  if constexpr (PF > 0) {
    const int live = static_cast<int>(row_hi - row_lo);
    const int slot = uw * (96 / NW) + lane % (96 / NW);  // 96 rows over the wavefronts
    if (slot < BM / 8) {
      int r = (nt % 8) * (BM / 8) + slot;
      r = r < live ? r : live - 1;
      pf_ptr = p.a + (row_lo + r) * p.K;
    } else {
      pf_ptr = bmat + (n0 + (mt % 4) * (BN / 4) + (slot - BM / 8) % (BN / 4)) * p.K;
    }
  }
  auto prefetch = [&](int kb) {
    if constexpr (PF > 0) dma4(pf_ptr + static_cast<int64_t>(kb_begin + kb) * 128, lds_addr(s_filler));
  };
  constexpr int ND = A_DMA + B_DMA;  // tile DMAs per wavefront per stage
  // The fp32-scale dense tiles with block scales issue each DMA right after
  // one MFMA (the interleaved issue described in the K loop).
  constexpr bool ILV_DENSE = !GROUPED && !SCALED && !EXACT && !ROWS && BALIGN && NW == 8;
  // Sub-tile steps that issue the DMAs: four of eight for those tiles (their
  // GEMM on 4096 x 7168 x 7168: 187.9 us over six steps, 185.7 over four, 185.3
  // over two, 188.7 in one), six of eight for the other 256 x 256 tiles, three
  // of four for the grouped ones (1.6% faster on the MoE shape than two, which
  // the row-scaled weight-gradient tiles keep: three is 1-8% slower there)
  constexpr int SPREAD = ILV_DENSE ? 4 : (SN >= 7 ? SN - 2 : (SN >= 4 ? (GROUPED ? SN - 1 : SN / 2) : SN));
  auto dma_tile = [&](int d, int kb, int st) {
    const int64_t kof = static_cast<int64_t>(kb_begin + kb) * 128;
    const uint32_t so = static_cast<uint32_t>(st) * STAGE;
    if (d < A_DMA) {
      if constexpr (GATHER)
        dma16_masked(a_base + kof, va[d], lds_ta + so + d * 1024, a_live[d]);
      else
        dma16_masked(a_base + kof + static_cast<int64_t>(d) * 8 * p.K, voff, lds_ta + so + d * 1024, a_live[d]);
    } else if constexpr (!B_RR) {
      dma16(b_base + kof + static_cast<int64_t>(d - A_DMA) * 8 * p.K, voff, lds_tb + so + (d - A_DMA) * 1024);
    } else {
      const int db = d - A_DMA;
      dma16_masked(b_base + kof + static_cast<int64_t>(db) * NW * 8 * p.K, voff, lds_tb + so + db * NW * 1024,
                   uw + NW * db < B_GROUPS ? ~0ull : 0ull);
    }
  };
  auto dma_scale = [&](int kb, int st) {
    dma4(gs + kb_begin + kb, lds_s0 + static_cast<uint32_t>(st) * lds_s_step);
    if constexpr (SB_EXTRA) {
      if (uwave == 0) dma4(gsb + kb_begin + kb, lds_addr(&s_sb[0][0]) + static_cast<uint32_t>(st) * (SB_LEN * 4));
    }
  };
  auto issue = [&](int kb, int st) {
#pragma unroll
    for (int d = 0; d < ND; ++d) dma_tile(d, kb, st);
    dma_scale(kb, st);
  };

  v4f acc[SN][SM];  // (a wavefront with fewer live row sub-tiles uses the first SMW columns)
#pragma unroll
  for (int i = 0; i < SN; ++i)
#pragma unroll
    for (int j = 0; j < SM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int KB = kb_count;  // K blocks this workgroup multiplies (from kb_begin)
  auto clampkb = [&](int kb) { return kb < KB ? kb : KB - 1; };
  {
    // Rows past the end of the expert's segment (or of the matrix) are never loaded: their LDS
    // slots are zeroed once here, so their MFMAs multiply zeros (which costs the
    // matrix cores far less power than the clamped copies of a real row would)
    // and their outputs, never stored, are zero.
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      if (!((a_live[i] >> lane) & 1)) {
#pragma unroll
        for (int s0 = 0; s0 < STAGES; ++s0)
          *reinterpret_cast<u32x4*>(tiles + s0 * STAGE + (wave * (BM / NW) + i * 8) * 128 + lane * 16) =
              u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // prologue: blocks 0 .. STAGES-2 into stages 0 .. STAGES-2
#pragma unroll
  for (int s0 = 0; s0 < STAGES - 1; ++s0) issue(clampkb(s0), s0);
  constexpr int PF_PRO = PF > STAGES ? PF - STAGES : 0;  // blocks STAGES .. PF-1, before the loop's
#pragma unroll
  for (int q = 0; q < PF_PRO; ++q) prefetch(clampkb(STAGES + q));
  // (loads complete in order: waiting for all but the newest PF_PRO retires block 0's DMAs)
  wait_barrier<WAIT_N + PF_PRO>();  // block 0 resident

  // Fragments of the current block: all m sub-tiles, the first n sub-tile, and
  // the per-column promotion factors sa[m,kb] * sb[nb,kb] (block mode) or sa[m,kb]
  // (row mode, where sb[n,kb] is read per n sub-tile); block 0 here, and the
  // loop requests each next block's right after its barrier.
  // A wavefront whose rows all lie past the end of the segment (or of the
  // matrix) has no product to form: it only issues its share of the tile loads
  // and meets the barriers, so the SIMD it shares runs the other wavefront's
  // MFMAs alone.
  // The wavefront's part of the tile: SMW row sub-tiles from tile row roff
  // (SMW = SM except for grouped tiles, below).
  auto body = [&](auto smc, const int roff) {
    constexpr int SMW = decltype(smc)::value;
    constexpr int TMW = SMW * 16;
    const bool wave_live = __builtin_amdgcn_readfirstlane(static_cast<int>(row_lo + roff < row_hi)) != 0;
    if (!wave_live) {
      int st = 0;
      for (int kb = 0; kb < KB; ++kb) {
        const int st_fill = st == 0 ? STAGES - 1 : st - 1;
        const int kb_fill = clampkb(kb + STAGES - 1);
#pragma unroll
        for (int d = 0; d < ND; ++d) dma_tile(d, kb_fill, st_fill);
        if (STAGES > 2 || uwave < SA_WAVES + SB_WAVES) dma_scale(kb_fill, st_fill);
        prefetch(clampkb(kb + PF));
        wait_barrier<WAIT_N + (PF > 0 ? 1 : 0)>();
        st = st == STAGES - 1 ? 0 : st + 1;
      }
    } else {
    v8i fm[SMW];
    float f[SMW];
    // Grouped tiles read each n fragment two sub-tile steps ahead (fn1 holds the
    // next one): 2% faster on the MoE shape, where a step is 4 MFMAs; the dense
    // tiles read one step ahead (two ahead measured 1.5% slower with eight
    // wavefronts and 18% slower with four).
    constexpr bool FD2 = GROUPED && SN > 2;
    v8i fn, fn1;
    // Scaled mode: E8M0 codes (the fp32 exponent field) of the lane's act-row
    // scale in each m sub-tile, and of the wavefront's weight-block scale.
    int ex[SMW];
    int ew = 0;
    auto e8m0 = [](float v) { return static_cast<int>((__float_as_uint(v) >> 23) & 0xFFu); };
    auto act_scale = [&](int st, int j) { return s_sa[st][roff + j * 16 + (lane & 15)]; };
    auto wgt_scale = [&](int st) { return s_sb[st][((wn * TN) / 128) % SB_LEN]; };
    // acc += 2^(ew-127) * 2^(ex-127) * (128-K FP8 partial), in one instruction; MFMA
    // "A" is the weight fragment (scale per weight row), "B" the act fragment.
    auto mma_scaled = [](const v8i& wfrag, const v8i& afrag, const v4f& c, int ewv, int exv) {
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfrag, afrag, c, 0, 0, 0, ewv, 0, exv);
    };
    auto factor = [&](int st, int j) {
      const float a = s_sa[st][roff + j * 16 + (lane & 15)];
      if constexpr (ROWS || !BALIGN)
        return a;
      else
        return a * s_sb[st][(wn * TN) / 128];
    };
    // Unaligned weight tiles: the block scale of n sub-tile i (staged blocks start
    // at block n0/128).
    const int n0_in_blk = static_cast<int>(n0 % 128);
    auto sub_scale = [&](int st, int i) { return s_sb[st][((n0_in_blk + wn * TN + i * 16) / 128) % SB_LEN]; };
    float sbv[BALIGN ? 1 : SN];
    // Row mode: the 4 weight-row scales of this lane in n sub-tile i.
    auto row_scales = [&](int st, int i) {
      return *reinterpret_cast<const v4f*>(&s_sb[st][(wn * TN + i * 16 + 4 * (lane >> 4)) % SB_LEN]);
    };
    // FP8 and scaled tiles read a block's fragments n first: after each barrier
    // the next block's n fragment and scales go out first, then its m
    // fragments, one right after each MFMA of the current block's last step, so
    // the next block's first MFMAs wait only for the reads they use.  The reads
    // before the loop take the same order: the compiler's waits at the loop
    // head merge both paths and would otherwise drain every read there.  In
    // one process with alternating blocks: dense 4096 x 7168 x 7168 in the step
    // 184.3 -> 183.4 us, power-of-two 166.7 -> 165.3 us, gathering MoE GEMM
    // 1376.6 -> 1370.5 us, outputs bit-identical.  The exact and row-scaled
    // tiles were slower (weight gradient 1549 -> 1607 and 1060 -> 1066 us) and
    // keep the former order.
    constexpr bool NFIRST = !EXACT && !ROWS;
    // The block in stage st: n fragment(s) and scales, then m fragment j right
    // after before_fm(j) (an MFMA of the last step, or nothing before the loop).
    auto read_block_nfirst = [&](int st, auto before_fm) {
      const uint8_t* tA = tiles + st * STAGE;
      const v8i n0 = frag(tA + TILE_A, wn * TN, lane);
      v8i n1;
      if constexpr (FD2) n1 = frag(tA + TILE_A, wn * TN + 16, lane);
      float sa_v[SMW];
#pragma unroll
      for (int j = 0; j < SMW; ++j) sa_v[j] = act_scale(st, j);
      const float sw_v = wgt_scale(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        before_fm(j);
        // (After the final block this reads a stage nobody uses; the values are dropped.)
        fm[j] = frag(tA, roff + j * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        if constexpr (SCALED)
          ex[j] = e8m0(sa_v[j]);
        else if constexpr (BALIGN)
          f[j] = sa_v[j] * sw_v;
        else
          f[j] = sa_v[j];
      }
      if constexpr (SCALED) ew = e8m0(sw_v);
      fn = n0;
      if constexpr (FD2) fn1 = n1;
    };
    if constexpr (NFIRST) {
      read_block_nfirst(0, [](int) {});
    } else {
      const uint8_t* tA = tiles;
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        fm[j] = frag(tA, roff + j * 16, lane);
        f[j] = factor(0, j);
      }
      fn = frag(tA + TILE_A, wn * TN, lane);
      if constexpr (FD2) fn1 = frag(tA + TILE_A, wn * TN + 16, lane);
    }

    // 128-K partial of n sub-tile `b` and m sub-tile `a` (MFMA A = weight rows).
    WideFrag wm_frag[EXACT ? SMW : 1];
    auto partial = [&](const v8i& b, const WideFrag& wb, int j) {
      const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (!EXACT) {
        (void)wb;
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, fm[j], z, 0, 0, 0, 0, 0, 0);
      } else {
        (void)b;
        v4f r = z;
#pragma unroll
        for (int q = 0; q < 4; ++q) r = __builtin_amdgcn_mfma_f32_16x16x32_f16(wb.q[q], wm_frag[j].q[q], r, 0, 0, 0);
        return r;
      }
    };
    // acc[i] += P * factor, with the row scales of sub-tile i in row mode, or the
    // block scale bs of sub-tile i for unaligned weight tiles.
    auto promote = [&](v4f* a, const v4f (&P)[SMW], const float (&fv)[SMW], const v4f& sbr, float bs) {
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        const float fj = BALIGN ? fv[j] : fv[j] * bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (ROWS)
            a[j][r] = fmaf(P[j][r] * sbr[r], fv[j], a[j][r]);
          else
            a[j][r] = fmaf(P[j][r], fj, a[j][r]);
        }
      }
    };
    auto bsv = [&](int i) { if constexpr (BALIGN) return 0.0f; else return sbv[i]; };

    int st = 0;  // stage holding block kb
    v4f P[2][SMW];
    v4f sbr[2];  // row mode: row scales of the sub-tiles whose partials are pending
    // Grouped tiles: the last sub-tile's partials are formed right after the
    // barrier; promoting them at once would wait on those MFMAs (s_nop hazards).
    // Their promotion is deferred to the first sub-tile step of the next block,
    // with the block's factors kept in f_prev (P[(SN-1)&1] and sbr[(SN-1)&1] are
    // not rewritten before then: step 0 writes the other buffer).  1.8% faster on
    // the MoE shape; 1% slower on the dense 256 x 256 tile, which keeps the
    // immediate promotion.
    constexpr bool DEFER = GROUPED && !SCALED && BALIGN;
    static_assert(!DEFER || SN % 2 == 0, "the deferred partials use the buffer step 0 does not write");
    // Interleaved issue (the four-wavefront power-of-two tiles, the grouped FP8
    // tiles and the fp32-scale dense tiles with block scales): the step's tile
    // DMAs are not issued together before its MFMAs but one after each MFMA,
    // followed (fp32 scales) by the promotion of the previous step's partial
    // for the same m sub-tile, in an order fixed by scheduling barriers.  A
    // wavefront issues in order, so a run of DMA instructions (each with its M0
    // write and wait state) behind a run of MFMAs leaves the matrix core idle
    // once the MFMAs drain; alone on its SIMD, nothing else fills that gap.
    // Dense 4096 x 7168 x 7168 with power-of-two scales 176.3 -> 169.0 and
    // 179.0 -> 171.9 us (two boxes), the gathering MoE GEMM 1421.9 -> 1397.1
    // us, outputs bit-identical.  The fp32-scale dense tiles gain only together
    // with an earlier DMA spread (four steps instead of six: 188.8 -> 187.4 and
    // 187.9 -> 185.7 us; with six, 189.3 vs 189.5).  The exact tiles (weight
    // gradient 1609 vs 1630 us) gain nothing and keep the compiler's order.
    constexpr bool ILV = (SCALED && NW == 4) || (GROUPED && !SCALED && !EXACT) || ILV_DENSE;
    static_assert(!ILV || SCALED || !ROWS, "the interleaved promotion is the block-scale form");
    static_assert(!ILV || PF == 0 || SPREAD <= SN - 2, "the L2 prefetch stays each iteration's newest load");
    float f_prev[SMW];
    for (int kb = 0; kb < KB; ++kb) {
      // Block kb+STAGES-1 goes into the stage consumed in the previous iteration.
      // Near the end the free stage is refilled with block KB-1, which is not read
      // again: the loop body stays branch-free and every wait is the same.
      const int st_fill = st == 0 ? STAGES - 1 : st - 1;
      const int kb_fill = clampkb(kb + STAGES - 1);
      // Interleaved issue: the j-th tile DMA of step i, if that step has one.
      auto dma_slot = [&](int i, int j) {
        const int d = i * ND / SPREAD + j;
        if (i < SPREAD && d < (i + 1) * ND / SPREAD) dma_tile(d, kb_fill, st_fill);
      };
      const uint8_t* tB = tiles + st * STAGE + TILE_A;
      if constexpr (!BALIGN) {
#pragma unroll
        for (int i = 0; i < SN; ++i) sbv[i] = sub_scale(st, i);
      }
      if constexpr (EXACT) {
#pragma unroll
        for (int j = 0; j < SMW; ++j) wm_frag[j] = widen(fm[j]);
      }
      __builtin_amdgcn_s_setprio(1);  // the issuing phase of the matrix cores goes first
      // Sub-tile steps 0 .. SN-2: the fragment of step i+1 is read from LDS while
      // the MFMAs of step i run, and the promotion FMAs of step i-1 (double-
      // buffered partials) fill the VALU under them.
#pragma unroll
      for (int i = 0; i < SN - 1; ++i) {
        // The loads of the block being prefetched go out over the first SPREAD
        // sub-tile steps, between MFMAs.
        if (!ILV && i < SPREAD) {
#pragma unroll
          for (int d = i * ND / SPREAD; d < (i + 1) * ND / SPREAD; ++d) dma_tile(d, kb_fill, st_fill);
        }
        if (i == 0) {
          // With two stages every wait drains all loads, so the filler DMAs that
          // keep the per-wavefront load count uniform are only needed with more.
          if (STAGES > 2 || uwave < SA_WAVES + SB_WAVES) dma_scale(kb_fill, st_fill);
        }
        if (i == SN - 2) prefetch(clampkb(kb + PF));  // after this iteration's DMAs
        v8i fn_next;  // the fragment this step reads: step i + 1's, or i + 2's with FD2
        if constexpr (FD2) {
          if (i + 2 < SN) fn_next = frag(tB, wn * TN + (i + 2) * 16, lane);
        } else {
          fn_next = frag(tB, wn * TN + (i + 1) * 16, lane);
        }
        if constexpr (ROWS) sbr[i & 1] = row_scales(st, i);
        if constexpr (SCALED) {
          const int ewi = BALIGN ? ew : e8m0(bsv(i));
#pragma unroll
          for (int j = 0; j < SMW; ++j) {
            acc[i][j] = mma_scaled(fn, fm[j], acc[i][j], ewi, ex[j]);
            if constexpr (ILV) {
              dma_slot(i, j);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else if constexpr (ILV) {
          const WideFrag none{};
#pragma unroll
          for (int j = 0; j < SMW; ++j) {
            P[i & 1][j] = partial(fn, none, j);
            dma_slot(i, j);
            if (i > 0) {
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = fmaf(P[(i - 1) & 1][j][r], f[j], acc[i - 1][j][r]);
            } else if (DEFER && kb > 0) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[SN - 1][j][r] = fmaf(P[(SN - 1) & 1][j][r], f_prev[j], acc[SN - 1][j][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          WideFrag wn_frag;
          if constexpr (EXACT) wn_frag = widen(fn);
#pragma unroll
          for (int j = 0; j < SMW; ++j) P[i & 1][j] = partial(fn, wn_frag, j);
          if constexpr (!GROUPED && (EXACT || !ROWS)) {
            // Tie the previous step's partials to this point: without it the
            // compiler promotes each partial right after its own MFMA (fewer
            // live registers) and the FMAs wait on the matrix core (s_nop);
            // here they read results four MFMAs old.  Dense 4096 x 7168 x 7168
            // 193.4 -> 190.6 us, exact weight gradient 1630 -> 1586 us; no gain
            // on the grouped or the row-scaled FP8 tiles, which keep the
            // compiler's order.
            if (i > 0) {
#pragma unroll
              for (int j = 0; j < SMW; ++j) asm volatile("" : "+v"(P[(i - 1) & 1][j]));
            }
          }
          if (i > 0)
            promote(acc[i - 1], P[(i - 1) & 1], f, sbr[(i - 1) & 1], bsv(i > 0 ? i - 1 : 0));
          else if (DEFER && kb > 0)
            promote(acc[SN - 1], P[(SN - 1) & 1], f_prev, sbr[(SN - 1) & 1], 0.0f);
        }
        if constexpr (ILV) {
          // the step's DMAs beyond its MFMA count (grouped tiles with few live rows)
          if (i < SPREAD) {
#pragma unroll
            for (int d = i * ND / SPREAD + SMW; d < (i + 1) * ND / SPREAD; ++d) dma_tile(d, kb_fill, st_fill);
          }
        }
        if constexpr (FD2) {
          fn = fn1;
          if (i + 2 < SN) fn1 = fn_next;
        } else {
          fn = fn_next;
        }
      }
      if constexpr (ROWS) sbr[(SN - 1) & 1] = row_scales(st, SN - 1);

      // Every LDS read of this stage has been issued: once they have returned and
      // block kb+1 is resident, the workgroup synchronises.  The last step's MFMAs
      // run after the barrier, and the next block's fragments are requested as
      // each m fragment is consumed, so their LDS latency hides under the MFMAs.
      __builtin_amdgcn_s_setprio(0);
      // the newest load, this iteration's prefetch, may stay in flight
      wait_barrier<WAIT_N + (PF > 0 ? 1 : 0)>();
      st = st == STAGES - 1 ? 0 : st + 1;
      if constexpr (SCALED) {
        const int ew_old = BALIGN ? ew : e8m0(bsv(SN - 1));
        const v8i fn_old = fn;
        int ex_old[SMW];
#pragma unroll
        for (int j = 0; j < SMW; ++j) ex_old[j] = ex[j];
        read_block_nfirst(st, [&](int j) { acc[SN - 1][j] = mma_scaled(fn_old, fm[j], acc[SN - 1][j], ew_old, ex_old[j]); });
        continue;
      }
      float f_old[SMW];
#pragma unroll
      for (int j = 0; j < SMW; ++j) f_old[j] = f[j];
      if constexpr (NFIRST) {
        const v8i fn_old = fn;
        const WideFrag none{};
        read_block_nfirst(st, [&](int j) { P[(SN - 1) & 1][j] = partial(fn_old, none, j); });
      } else {
        const uint8_t* tA = tiles + st * STAGE;
        WideFrag wn_frag;
        if constexpr (EXACT) wn_frag = widen(fn);
#pragma unroll
        for (int j = 0; j < SMW; ++j) {
          P[(SN - 1) & 1][j] = partial(fn, wn_frag, j);
          // (After the final block this reads a stage nobody uses; the values are dropped.)
          fm[j] = frag(tA, roff + j * 16, lane);
          f[j] = factor(st, j);
        }
        fn = frag(tA + TILE_A, wn * TN, lane);
        if constexpr (FD2) fn1 = frag(tA + TILE_A, wn * TN + 16, lane);
      }
      promote(acc[SN - 2], P[(SN - 2) & 1], f_old, sbr[(SN - 2) & 1], bsv(SN - 2));
      if constexpr (DEFER) {
#pragma unroll
        for (int j = 0; j < SMW; ++j) f_prev[j] = f_old[j];
      } else {
        promote(acc[SN - 1], P[(SN - 1) & 1], f_old, sbr[(SN - 1) & 1], bsv(SN - 1));
      }
    }
    if constexpr (DEFER) {
      if (KB > 0) promote(acc[SN - 1], P[(SN - 1) & 1], f_prev, sbr[(SN - 1) & 1], 0.0f);
    }
    }  // live wavefront
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA may outlive the workgroup

    // ---- epilogue: lane holds Y[m][n .. n+3], m = sub-tile column, n = 4 consecutive rows
    __syncthreads();  // every wavefront is done with the tile buffers
    if constexpr (QOUT != 0) {
      // The wavefront's 128 columns of a row are one 1x128 group.  Row m = j*16 +
      // (lane & 15) of sub-tile column j sits in lanes l, l^16, l^32, l^48, 32
      // values each: amax over the lane's values, then over those four lanes.
      // Codes are staged in LDS as 128-byte rows and leave as whole rows.
      constexpr int QP = 128 + 16;  // staging pitch (bytes)
      static_assert(NW * TM * QP <= TILES_BYTES, "staging fits the tile buffers");
      uint8_t* epi = tiles + wave * TM * QP;
      const int64_t gcol = (n0 + wn * TN) / 128;  // group index along N
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < SN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(acc[i][j][r]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        float sc, inv;
        group_scale<QOUT == 2>(am, sc, inv);
        const int mr = j * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < SN; ++i)
          *reinterpret_cast<uint32_t*>(epi + mr * QP + i * 16 + 4 * (lane >> 4)) =
              cvt4(acc[i][j][0] * inv, acc[i][j][1] * inv, acc[i][j][2] * inv, acc[i][j][3] * inv);
        const int64_t m = row_lo + roff + mr;
        if (lane < 16 && m < row_hi) p.ys[m * (p.N / 128) + gcol] = sc;
      }
      // (ds ops of one wavefront complete in order: no barrier needed here)
#pragma unroll
      for (int pass = 0; pass < TMW / 8; ++pass) {
        const int mr = pass * 8 + lane / 8;
        const int64_t m = row_lo + roff + mr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(epi + mr * QP + (lane % 8) * 16);
        if (m < row_hi)
          *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.y) + m * p.N + n0 + wn * TN + (lane % 8) * 16) = v;
      }
    } else if constexpr (BF16OUT) {
      // Stage the wavefront's TM x TN block as bf16 rows in LDS (8 bytes per lane
      // and sub-tile), then write whole row segments (TN*2 bytes = 16 lanes x 16 B).
      uint8_t* epi = tiles + wave * TM * EPI_PITCH;
#pragma unroll
      for (int j = 0; j < SMW; ++j)
#pragma unroll
        for (int i = 0; i < SN; ++i) {
          const int mr = j * 16 + (lane & 15);
          const int nc = i * 16 + 4 * (lane >> 4);
          u32x2 o;
          o[0] = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
          o[1] = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<u32x2*>(epi + mr * EPI_PITCH + nc * 2) = o;
        }
      // (ds ops of one wavefront complete in order: no barrier needed here)
      constexpr int LANES_PER_ROW = TN * 2 / 16;
      constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
      static_assert(TMW % ROWS_PER_PASS == 0, "whole passes");
      const int c16 = lane % LANES_PER_ROW;
      const bool epi_lane = lane < ROWS_PER_PASS * LANES_PER_ROW;
#pragma unroll
      for (int pass = 0; pass < TMW / ROWS_PER_PASS; ++pass) {
        const int mr = pass * ROWS_PER_PASS + (epi_lane ? lane / LANES_PER_ROW : 0);
        const int64_t m = row_lo + roff + mr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(epi + mr * EPI_PITCH + c16 * 16);
        if (epi_lane && m < row_hi)
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.y) + m * p.N + n0 + wn * TN + c16 * 8) = v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < SMW; ++j) {
        const int64_t m = row_lo + roff + j * 16 + (lane & 15);
        if (m >= row_hi) continue;
#pragma unroll
        for (int i = 0; i < SN; ++i) {
          const int64_t n = n0 + wn * TN + i * 16 + 4 * (lane >> 4);
          float* dst = static_cast<float*>(p.y) + m * p.N + n;
          if (add_out) {
            // K-split part: add into the zeroed output (hardware fp32 atomics)
#pragma unroll
            for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dst + r, acc[i][j][r]);
          } else {
            *reinterpret_cast<v4f*>(dst) = acc[i][j];
          }
        }
      }
    }
  };
  if constexpr (GROUPED) {
    // Only the row sub-tiles that hold rows of the segment are multiplied: the
    // K loop is compiled for 1 .. SM sub-tiles and each wavefront runs the copy
    // for its live rows (chosen once per tile; no branch inside the loop).  The
    // last m-tile of every expert segment is partial, and multiplying its rows
    // past the segment end cost 12% more FP8 work than the segments hold.
    const int64_t live64 = row_hi - (row_lo + wm * TM);
    const int live = __builtin_amdgcn_readfirstlane(static_cast<int>(live64 < 0 ? 0 : (live64 > TM ? TM : live64)));
    const int smw = (live + 15) / 16;  // 0: no live row (the copy for one sub-tile, whose loop it skips)
    auto pick = [&](auto self, auto kc) -> void {
      constexpr int k = decltype(kc)::value;
      if constexpr (k == 1) {
        body(kc, wm * TM);
      } else {
        if (smw >= k)
          body(kc, wm * TM);
        else
          self(self, std::integral_constant<int, k - 1>{});
      }
    };
    pick(pick, std::integral_constant<int, SM>{});
  } else {
    body(std::integral_constant<int, SM>{}, wm * TM);
  }
}

// Tile configurations: {BM, BN, WM, WN, STAGES}.
//   0: 256 x 256, 4 x 2 wavefronts (64 x 128 each), 2 stages (128 KB LDS)
//   1: 128 x 256, 2 x 4 wavefronts (64 x 64 each), 3 stages (144 KB LDS)
//   2: 256 x 224, 4 x 2 wavefronts (64 x 112 each), 2 stages (120 KB LDS)
//   3: 256 x 256, 2 x 2 wavefronts (128 x 128 each, one per SIMD), 2 stages:
//      scaled mode only, where the 256 accumulators per lane sit in AGPRs and
//      the matrix cores accumulate into them directly (with fp32 scales the
//      promotion would have to move every accumulator through VGPRs: 22% slower)
template <int CFG> struct Cfg;
template <> struct Cfg<0> { static constexpr int BM = 256, BN = 256, WM = 4, WN = 2, ST = 2; };
template <> struct Cfg<1> { static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, ST = 3; };
template <> struct Cfg<2> { static constexpr int BM = 256, BN = 224, WM = 4, WN = 2, ST = 2; };
template <> struct Cfg<3> { static constexpr int BM = 256, BN = 256, WM = 2, WN = 2, ST = 2; };

// Zeroes the fp32 output of the K-split tiles (tiles T_full .. T_full +
// gridDim.x - 1 of the dense order) before their parts add into it.  A kernel,
// not a memset, so the sequence can be captured in a graph.
template <int BM, int BN>
__global__ void __launch_bounds__(256) zero_split_tiles_kernel(float* __restrict__ y, int64_t M, int64_t N, int MT,
                                                               int NT, int T_full) {
  int mt, nt;
  dense_tile_coords(T_full + static_cast<int>(blockIdx.x), MT, NT, mt, nt);
  const int64_t r0 = static_cast<int64_t>(mt) * BM, c0 = static_cast<int64_t>(nt) * BN;
  for (int idx = threadIdx.x; idx < BM * (BN / 4); idx += 256) {
    const int r = idx / (BN / 4), c = idx % (BN / 4);
    if (r0 + r < M) *reinterpret_cast<v4f*>(y + (r0 + r) * N + c0 + 4 * c) = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
}

// Compute units of the current device, queried once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int CFG, bool EXACT, bool ROWS, bool BF16OUT, bool GROUPED, bool GATHER, bool SCALED, int QOUT = 0>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  using C = Cfg<CFG>;
  const int64_t MT = GROUPED ? g.M / C::BM + g.G : (g.M + C::BM - 1) / C::BM;
  FParams p{g.a, g.sa, g.b, g.sb, g.y, g.offsets, g.row_index, g.M, g.N, g.K, g.G, g.T,
            static_cast<int>(g.K / 128), static_cast<int>(MT), static_cast<int>(g.N / C::BN), g.y_scales};
  const int64_t T = MT * p.NT;
  p.T_full = static_cast<int>(T);
  p.split = 1;
  if constexpr (!GROUPED && !BF16OUT && QOUT == 0) {
    // fp32 output filling at least one round of the CUs: the tiles of the
    // partial last round are split along K over the CUs that round would leave
    // idle (the weight-gradient shape 7168 x 7168 has 1568 tiles of 128 x 256,
    // 6.125 rounds of 256 CUs; its last 32 tiles run as 8 parts each).  The
    // parts add in whatever order they finish, so those tiles' last bits can
    // differ between runs.  Smaller problems are not split, which keeps their
    // results equal bit for bit to the same sums computed by other tile shapes
    // (the grouped and the output-quantising kernels).
    const int ncu = device_cus();
    if (ncu > 0 && T >= ncu) {
      const int64_t full = (T / ncu) * ncu, rest = T - full;
      int64_t parts = rest > 0 ? ncu / rest : 1;
      parts = parts < p.KB ? parts : p.KB;
      if (parts >= 2) {
        p.T_full = static_cast<int>(full);
        p.split = static_cast<int>(parts);
        hipLaunchKernelGGL((zero_split_tiles_kernel<C::BM, C::BN>), dim3(static_cast<unsigned>(rest)), dim3(256), 0,
                           s, static_cast<float*>(g.y), g.M, g.N, p.MT, p.NT, p.T_full);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  const unsigned blocks = static_cast<unsigned>(p.T_full + (T - p.T_full) * p.split);
  hipLaunchKernelGGL(
      (gemm_fp8_block_kernel<C::BM, C::BN, C::WM, C::WN, C::ST, EXACT, ROWS, BF16OUT, GROUPED, GATHER, SCALED,
                             QOUT>),
      dim3(blocks), dim3(C::WM * C::WN * 64), 0, s, p);
  return hipGetLastError();
}

template <int CFG, bool EXACT, bool ROWS, bool GROUPED, bool GATHER = false, bool SCALED = false>
hipError_t launch_out(const GemmArgs& g, hipStream_t s) {
  return g.y_bf16 ? launch_cfg<CFG, EXACT, ROWS, true, GROUPED, GATHER, SCALED>(g, s)
                  : launch_cfg<CFG, EXACT, ROWS, false, GROUPED, GATHER, SCALED>(g, s);
}

}  // namespace

bool fp8_block_kernel_applies(const GemmArgs& g) {
  // (the DMA lane offsets are 32-bit: 256 rows x K bytes must stay below 4 GiB)
  if (g.K >= (int64_t(1) << 24)) return false;
  if (g.N % 256 == 0) return true;
  // 224-wide tiles: dense, 128x128 weight scales, FP8 or scaled accumulation
  return g.N % 224 == 0 && g.offsets == nullptr && !g.exact && !g.row_scales;
}

namespace {

// Width of the 256-row dense tiles: 256 whenever N allows it, else 224.
// Measured on 4096 x 7168 x 7168, 224-wide tiles (512 tiles, exactly two
// rounds of the 256 CUs) run 5-8% slower than 256-wide ones (448 tiles, 1.75
// rounds): the per-block costs (barrier, A fragments, scales) are spread over
// 7/8 of the MFMAs, and the last round of 256-wide tiles runs on a partly idle
// chip at a higher clock.  So 224 serves only N that 256 does not divide.
int dense_tile_width(const GemmArgs& g) { return g.N % 256 == 0 ? 256 : 224; }

}  // namespace

// Block-scaled FP8 accumulation: dense GEMMs use the 256 x 256 tile (least L2
// and LDS traffic per flop), grouped GEMMs the 128-row tile (expert segments of
// ~256 rows then waste less of their last m-tile).  The exact mode (fp16
// operands, twice the fragment registers) uses the 64 x 64 wavefront tile; the
// row-scaled FP8 mode (one more multiply and four row scales per sub-tile) the
// dense 256 x 256 tile.
// The scaled mode (power-of-two scales applied by the matrix cores) takes the
// same tiles as the FP8 mode.
hipError_t launch_grouped_gemm_gather(const GemmArgs& g, hipStream_t s) {
  if (g.scaled) return launch_out<1, false, false, true, true, true>(g, s);
  return g.exact ? launch_out<1, true, false, true, true>(g, s) : launch_out<1, false, false, true, true>(g, s);
}

hipError_t launch_fp8_block_gemm(const GemmArgs& g, bool grouped, hipStream_t s) {
  if (grouped) {
    if (g.scaled) return launch_out<1, false, false, true, false, true>(g, s);
    return g.exact ? launch_out<1, true, false, true>(g, s) : launch_out<1, false, false, true>(g, s);
  }
  if (g.exact)
    return g.row_scales ? launch_out<1, true, true, false>(g, s) : launch_out<1, true, false, false>(g, s);
  // Row-scaled B with FP8 accumulation fits the 256 x 256 tile (244 VGPRs with
  // the four row scales per sub-tile): 10% faster than 128 x 256 on the weight
  // gradient 7168 x 7168 x 16384.  Exact mode keeps 128 x 256 (its fp16
  // fragments need the registers).
  if (g.row_scales) return launch_out<0, false, true, false>(g, s);
  const bool narrow = dense_tile_width(g) == 224;
  // (scaled mode: four wavefronts of 128 x 128 on 256 x 256 tiles, 2.5% faster
  // than eight of 64 x 128 on 4096 x 7168 x 7168: half the fragment reads and
  // half the wavefronts at each barrier)
  if (g.scaled)
    return narrow ? launch_out<2, false, false, false, false, true>(g, s)
                  : launch_out<3, false, false, false, false, true>(g, s);
  return narrow ? launch_out<2, false, false, false>(g, s) : launch_out<0, false, false, false>(g, s);
}

// GEMM whose output leaves 1x128-quantised (256 x 256 dense tiles: a
// wavefront's 128 columns are one group).  FP8 or scaled accumulation.
hipError_t launch_fp8_block_gemm_quant(const GemmArgs& g, bool pow2, hipStream_t s) {
  // (the scaled mode keeps eight wavefronts here: with four, the quantising
  // epilogue needs more than the 512 registers of a wavefront and spills)
  if (g.scaled)
    return pow2 ? launch_cfg<0, false, false, false, false, false, true, 2>(g, s)
                : launch_cfg<0, false, false, false, false, false, true, 1>(g, s);
  return pow2 ? launch_cfg<0, false, false, false, false, false, false, 2>(g, s)
              : launch_cfg<0, false, false, false, false, false, false, 1>(g, s);
}

}  // namespace fp8fg
