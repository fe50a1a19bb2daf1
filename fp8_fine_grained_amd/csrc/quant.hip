// Online fine-grained quantisation to OCP E4M3 on gfx950.
//
// Per group (1x128 activation tile or 128x128 weight block; Figure 7(a)
// passage of the innerforce DeepSeek-V3 notes, yunhecapital report section
// 2.2.3, tonho.wtf "DeepSeek-V3" section "como funciona"):
//     amax = max|x|,  s = fl32(amax/448),  inv = s ? fl32(1/s) : 0,
//     q = E4M3 RNE cast of fl32(x*inv), sign kept.
// The divisions use HIP's correctly rounded fp32 division (no fast math).
// |x*inv| <= 448*(1+3*2^-24) < 464, so the hardware cvt, which rounds to
// nearest even and maps [448, 464] to 448, never reaches its NaN range and
// no explicit clamp is needed; zero groups give inv = 0 and codes 0x00/0x80.
//
// Power-of-two (E8M0) scales, for matrix cores that apply group scales
// themselves (the microscaling formats the innerforce notes' Figure 7(a)
// passage relates the grouping to; the group-scaled MMA of the tonho.wtf
// wish list, "o que isso custou"): s = 2^e with e the smallest integer such
// that amax <= 448 * 2^e, inv = 2^-e.  Writing amax = m * 2^E (m in [1, 2)),
// amax / 2^(E-8) = 256 m is within 448 unless m > 1.75, so e = E - 8, plus one
// when the mantissa field exceeds 0x600000 (m > 1.75).  x * inv is exact and
// |x * inv| <= 448.
#include "launch.h"
#include "quant_rule.h"

namespace fp8fg {
namespace {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));



// Codes are written with ordinary (cache-allocating) stores, inputs read with
// non-temporal loads: the GEMM that follows reads the codes, and stores that
// allocate keep them (X 29 MB + W 51 MB for the dense projection) in the 256 MB
// last-level cache, while the streamed bf16 inputs, read once, do not displace
// them.  Measured on the dense step against non-temporal code stores: GEMM 201
// -> 194 us, quantisers unchanged.
template <typename V>
__device__ __forceinline__ void store_codes(const V& v, void* p) {
  *reinterpret_cast<V*>(p) = v;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}
// Max over each aligned group of 8 lanes (quad xor 1, quad xor 2, half-row mirror).
__device__ __forceinline__ float max8(float v) {
  v = dpp_max<0xB1>(v);
  v = dpp_max<0x4E>(v);
  return dpp_max<0x141>(v);
}
// Max over the 64-lane wavefront.
__device__ __forceinline__ float max64(float v) {
  v = max8(v);
  v = dpp_max<0x140>(v);  // row mirror: max over 16
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

// Lane layout of a 128-element group row read by 8 lanes: lane `part` holds
// NR runs of L = 16 bytes / element size consecutive elements, run r starting
// at element r * 8L + part * L.  Each load instruction of the 8 lanes then
// reads 128 contiguous bytes (whole lines, the pattern the memory system
// serves fastest); a lane holding 16 consecutive elements would make each
// instruction read every other 16 bytes of 256 (bf16, 1x128 quantiser on
// [16384,7168]: 56.6 -> 54.1 us).  v[r * L + i] is element r * 8L + part * L + i.
template <bool BF16>
struct Runs {
  static constexpr int L = BF16 ? 8 : 4;  // elements per run
  static constexpr int NR = 16 / L;       // runs per lane
  static constexpr int ES = BF16 ? 2 : 4;
  // element index of run r of lane `part`
  static __device__ __forceinline__ int col(int r, int part) { return r * 8 * L + part * L; }
};

// The lane's 16 elements of the group row starting at `row` (16-byte aligned), as fp32.
template <bool BF16>
__device__ __forceinline__ void load_runs(const void* row, int part, float (&v)[16]) {
  using R = Runs<BF16>;
#pragma unroll
  for (int r = 0; r < R::NR; ++r) {
    const void* p = static_cast<const char*>(row) + R::col(r, part) * R::ES;
    if constexpr (BF16) {
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[r * 8 + 2 * i] = bf16_lo(w[i]);
        v[r * 8 + 2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
      v[r * 4] = t.x;
      v[r * 4 + 1] = t.y;
      v[r * 4 + 2] = t.z;
      v[r * 4 + 3] = t.w;
    }
  }
}

// The 16 codes of the lane (code dword d = elements 4d .. 4d+3 of v) into the
// group's 128-byte code row `dst`, each run's codes at the run's own columns.
template <bool BF16>
__device__ __forceinline__ void store_runs(const u32x4& c, uint8_t* dst, int part) {
  using R = Runs<BF16>;
  if constexpr (BF16) {
    store_codes(u32x2{c.x, c.y}, dst + R::col(0, part));
    store_codes(u32x2{c.z, c.w}, dst + R::col(1, part));
  } else {
    store_codes(c.x, dst + R::col(0, part));
    store_codes(c.y, dst + R::col(1, part));
    store_codes(c.z, dst + R::col(2, part));
    store_codes(c.w, dst + R::col(3, part));
  }
}

// ---------------------------------------------------------------- 1x128, rows
// Eight lanes own one 1x128 tile (16 elements each, in the run layout); a 256-thread block
// covers 32 consecutive tiles of the row-major [M, K/128] tile grid.
template <bool BF16, bool POW2>
__device__ __forceinline__ void act_rows_block(int64_t b, const void* __restrict__ x, int64_t ld, int G,
                                               int64_t tiles, uint8_t* __restrict__ q,
                                               float* __restrict__ scales, int64_t K) {
  const int64_t tile = b * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const bool live = tile < tiles;
  const int64_t t = live ? tile : tiles - 1;  // dead lanes mirror the last tile; they store nothing
  const int64_t m = t / G;
  const int g = static_cast<int>(t - m * G);
  const int64_t col = static_cast<int64_t>(g) * 128;
  constexpr int ES = BF16 ? 2 : 4;
  const char* src = static_cast<const char*>(x) + (m * ld + col) * ES;

  float v[16];
  load_runs<BF16>(src, part, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = max8(amax);
  float s, inv;
  group_scale<POW2>(amax, s, inv);
  u32x4 out;
  out.x = cvt4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  out.y = cvt4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  out.z = cvt4(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
  out.w = cvt4(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
  if (live) {
    store_runs<BF16>(out, q + m * K + col, part);
    if (part == 0) scales[t] = s;
  }
}

template <bool BF16, bool POW2>
__global__ void __launch_bounds__(256) quant_act_rows_kernel(const void* __restrict__ x, int64_t ld,
                                                             int G, int64_t tiles,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scales, int64_t K) {
  act_rows_block<BF16, POW2>(blockIdx.x, x, ld, G, tiles, q, scales, K);
}

// ---------------------------------------------------------------- per tensor
// One scale for the whole tensor, the practice the 1x128 / 128x128 grouping
// replaces (innerforce notes, Figure 7(a) passage), kept for the accuracy and
// cost comparison: the same rule with the amax taken over every element.
// Three launches and no workspace: (1) each block's amax into scales[b],
// (2) one block reduces them and stores s in scales[0], (3) the cast, which
// reads s from scales[0] and writes it into every other scale slot.

// (1) Blocks stride over 32-tile groups of the row-major [M, K/128] tile grid.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_pt_amax_kernel(const void* __restrict__ x, int64_t ld, int G,
                                                            int64_t tiles, float* __restrict__ partial) {
  __shared__ float wave_max[4];
  const int part = threadIdx.x & 7;
  constexpr int ES = BF16 ? 2 : 4;
  float amax = 0.0f;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 32; base < tiles;
       base += static_cast<int64_t>(gridDim.x) * 32) {
    const int64_t tile = base + (threadIdx.x >> 3);
    if (tile < tiles) {
      const int64_t m = tile / G;
      const int64_t col = (tile - m * G) * 128;
      float v[16];
      load_runs<BF16>(static_cast<const char*>(x) + (m * ld + col) * ES, part, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  amax = max64(amax);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[blockIdx.x] = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
}

// (2) One block: the amax of the n partial maxima, then s.
__global__ void __launch_bounds__(256) quant_pt_scale_kernel(float* __restrict__ scales, int n) {
  __shared__ float wave_max[4];
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) amax = fmaxf(amax, scales[i]);
  amax = max64(amax);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();  // every partial has been read before scales[0] is overwritten
  if (threadIdx.x == 0) {
    float s, inv;
    group_scale(fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3])), s, inv);
    scales[0] = s;
  }
}

// (3) The cast, laid out as the 1x128 row kernel; tile t also writes scale slot
// t (t in [1, n_scales)); slot 0 already holds s and is only read.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_pt_cast_kernel(const void* __restrict__ x, int64_t ld, int G,
                                                            int64_t tiles, uint8_t* __restrict__ q,
                                                            float* __restrict__ scales, int64_t n_scales, int64_t K) {
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  if (tile >= tiles) return;  // no cross-lane operations below
  const int64_t m = tile / G;
  const int64_t col = (tile - m * G) * 128;
  constexpr int ES = BF16 ? 2 : 4;
  const float s = scales[0];
  const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;  // as group_scale derives it from the same s
  float v[16];
  load_runs<BF16>(static_cast<const char*>(x) + (m * ld + col) * ES, part, v);
  u32x4 out;
  out.x = cvt4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  out.y = cvt4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  out.z = cvt4(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
  out.w = cvt4(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
  store_runs<BF16>(out, q + m * K + col, part);
  if (part == 0 && tile >= 1 && tile < n_scales) scales[tile] = s;
}

// ------------------------------------------------------- 1x128, transposed
// Input physically [K, ld] (e.g. tokens x channels); logical row m is column m,
// and a group is 128 consecutive physical rows (tokens) of one column.
// A 512-thread block handles one 128-row x 256-byte tile (128 bf16 or 64 fp32
// columns):
//  1. the tile is read with full 256-byte row segments (16 lanes per row) and
//     stored in LDS, the 16-byte chunks of row r XOR-permuted by
//     ((r >> 4) & 7) << 1;
//  2. thread (tg, d) reads dword d (2 bf16 / 1 fp32 columns) of rows
//     16*tg .. 16*tg+15 -- with the permutation, the 64 lanes of a wavefront hit
//     64 distinct banks -- reduces the amax over the 8 token groups of its
//     columns with DPP (the 8 groups are 8 consecutive lanes), and writes its
//     16 codes per column as one 16-byte store (8 threads write a column's 128
//     codes contiguously).
constexpr int kColsTileBytes = 256;
__device__ __forceinline__ int cols_swz(int row) { return ((row >> 4) & 7) << 1; }

template <bool BF16, bool POW2>
__global__ void __launch_bounds__(512) quant_act_cols_kernel(const void* __restrict__ x, int64_t ld,
                                                             int64_t M, int G, int CB,
                                                             uint8_t* __restrict__ q,
                                                             float* __restrict__ scales, int64_t K) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int COLS_PER_DW = BF16 ? 2 : 1;
  constexpr int TILE_COLS = kColsTileBytes / ES;
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kColsTileBytes];
  const int tid = threadIdx.x;
  // Token group fastest: consecutive blocks write adjacent 128-byte code runs of
  // the same 128 output rows (HBM pages are written whole; 79 -> 65 us on
  // [16384, 7168] bf16 against column block fastest, which scatters the writes).
  // Workgroup i runs on XCD i % 8, and each XCD takes one contiguous range of
  // that order, so the code runs and the 4-byte scales of an output row are
  // all written through one L2 (65 -> 62 us: neighbouring scales written from
  // different XCDs leave partly written lines in several L2s).
  const int nblk = static_cast<int>(gridDim.x);
  const int t = nblk % 8 == 0 ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
  const int g = t % G;   // token group
  const int cb = t / G;  // column block
  const int64_t col0 = static_cast<int64_t>(cb) * TILE_COLS;
  const int64_t row0 = static_cast<int64_t>(g) * 128;

  // 1. global -> LDS: thread t moves chunks (row t/16 + 32i, chunk t%16), i = 0..3.
  {
    const int c = tid & 15;
    int64_t ccol = col0 + c * (16 / ES);  // first column of the chunk
    const bool cvalid = ccol < M;         // M % 8 == 0: a chunk is all in or all out
    if (!cvalid) ccol = col0;             // stay inside the row; the data is never stored
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 32 * i;
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const char*>(x) + ((row0 + r) * ld + ccol) * ES));
      *reinterpret_cast<u32x4*>(tile + r * kColsTileBytes + ((c ^ cols_swz(r)) * 16)) = v;
    }
  }
  __syncthreads();

  // 2. thread (tg, d): the 8 token groups of a dword are 8 consecutive lanes;
  //    wavefront w owns dwords 8w .. 8w+7.
  const int lane = tid & 63;
  const int tg = lane & 7;                       // token group: rows 16*tg .. +15
  const int d = (tid >> 6) * 8 + (lane >> 3);    // dword of the 256-byte row, 0..63
  const int chunk = d >> 2, within = (d & 3) * 4;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * tg + i;
    w[i] = *reinterpret_cast<const uint32_t*>(tile + r * kColsTileBytes + ((chunk ^ cols_swz(r)) * 16) + within);
  }
  auto lo = [](uint32_t u) { return BF16 ? bf16_lo(u) : __uint_as_float(u); };
  float amax0 = 0.0f, amax1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax0 = fmaxf(amax0, fabsf(lo(w[i])));
    if constexpr (BF16) amax1 = fmaxf(amax1, fabsf(bf16_hi(w[i])));
  }
  // reduce over the 8 token groups (8 consecutive lanes: DPP, no LDS traffic)
  amax0 = max8(amax0);
  if constexpr (BF16) amax1 = max8(amax1);
  const int64_t m0 = col0 + static_cast<int64_t>(d) * COLS_PER_DW;
  if (m0 >= M) return;  // no cross-lane operations below
  float s0, inv0;
  group_scale<POW2>(amax0, s0, inv0);
  const int64_t k0 = row0 + 16 * tg;
  u32x4 o;
  o.x = cvt4(lo(w[0]) * inv0, lo(w[1]) * inv0, lo(w[2]) * inv0, lo(w[3]) * inv0);
  o.y = cvt4(lo(w[4]) * inv0, lo(w[5]) * inv0, lo(w[6]) * inv0, lo(w[7]) * inv0);
  o.z = cvt4(lo(w[8]) * inv0, lo(w[9]) * inv0, lo(w[10]) * inv0, lo(w[11]) * inv0);
  o.w = cvt4(lo(w[12]) * inv0, lo(w[13]) * inv0, lo(w[14]) * inv0, lo(w[15]) * inv0);
  store_codes(o, reinterpret_cast<u32x4*>(q + m0 * K + k0));
  if (tg == 0) scales[m0 * G + g] = s0;
  if constexpr (BF16) {
    float s1, inv1;
    group_scale<POW2>(amax1, s1, inv1);
    u32x4 h;
    h.x = cvt4(bf16_hi(w[0]) * inv1, bf16_hi(w[1]) * inv1, bf16_hi(w[2]) * inv1, bf16_hi(w[3]) * inv1);
    h.y = cvt4(bf16_hi(w[4]) * inv1, bf16_hi(w[5]) * inv1, bf16_hi(w[6]) * inv1, bf16_hi(w[7]) * inv1);
    h.z = cvt4(bf16_hi(w[8]) * inv1, bf16_hi(w[9]) * inv1, bf16_hi(w[10]) * inv1, bf16_hi(w[11]) * inv1);
    h.w = cvt4(bf16_hi(w[12]) * inv1, bf16_hi(w[13]) * inv1, bf16_hi(w[14]) * inv1, bf16_hi(w[15]) * inv1);
    store_codes(h, reinterpret_cast<u32x4*>(q + (m0 + 1) * K + k0));
    if (tg == 0) scales[(m0 + 1) * G + g] = s1;
  }
}

// ---------------------------------------------------------------- 128x128
// One 256-thread block per 128x128 block, read from HBM once: thread t holds
// columns 8*(t%16) .. +7 of rows t/16 + 16*i (i = 0..7) in registers.
template <bool BF16, bool POW2>
__device__ __forceinline__ void weight_block(int b, const void* __restrict__ w, int64_t ld, int GK,
                                             uint8_t* __restrict__ q, float* __restrict__ scales, int64_t K,
                                             float* wave_max) {
  const int bi = b / GK;
  const int bj = b - bi * GK;
  const int c8 = (threadIdx.x & 15) * 8;
  const int r0 = threadIdx.x >> 4;
  constexpr int ES = BF16 ? 2 : 4;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = static_cast<int64_t>(bi) * 128 + r0 + 16 * i;
    const char* src = static_cast<const char*>(w) + (row * ld + static_cast<int64_t>(bj) * 128 + c8) * ES;
    if constexpr (BF16) {
      u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[i][2 * j] = bf16_lo(wd[j]);
        v[i][2 * j + 1] = bf16_hi(wd[j]);
      }
    } else {
      f32x4 f0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
      f32x4 f1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + 1);
      v[i][0] = f0.x; v[i][1] = f0.y; v[i][2] = f0.z; v[i][3] = f0.w;
      v[i][4] = f1.x; v[i][5] = f1.y; v[i][6] = f1.z; v[i][7] = f1.w;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  amax = max64(amax);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  float s, inv;
  group_scale<POW2>(amax, s, inv);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = static_cast<int64_t>(bi) * 128 + r0 + 16 * i;
    u32x2 o;
    o.x = cvt4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
    o.y = cvt4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
    store_codes(o, reinterpret_cast<u32x2*>(q + row * K + static_cast<int64_t>(bj) * 128 + c8));
  }
  if (threadIdx.x == 0) scales[b] = s;
}

template <bool BF16, bool POW2>
__global__ void __launch_bounds__(256) quant_weight_kernel(const void* __restrict__ w, int64_t ld,
                                                           int GK, uint8_t* __restrict__ q,
                                                           float* __restrict__ scales, int64_t K) {
  __shared__ float wave_max[4];
  weight_block<BF16, POW2>(blockIdx.x, w, ld, GK, q, scales, K, wave_max);
}

// ------------------------------------------- 128x128 weight + 1x128 activation
// Both quantisers of a layer's step in one launch: workgroups 0 .. n_w-1 each
// quantise a 128x128 weight block, the rest 32 activation tiles each.  Two
// back-to-back launches each pay their own ramp and tail; one launch pays one,
// and with the longer weight blocks first the short activation blocks fill the
// tail (X [4096,7168] + W [7168,7168] bf16: 38.2 us against 42.9 us for the two
// launches).  Every code and scale equals the separate quantisers'.
struct ActWeightArgs {
  const void* x;
  int64_t ld_x, tiles, K_x;
  int G;
  uint8_t* q_x;
  float* s_x;
  const void* w;
  int64_t ld_w, K_w;
  int GK;
  uint8_t* q_w;
  float* s_w;
  int n_w;  // weight workgroups
};
template <bool XBF16, bool WBF16, bool POW2>
__global__ void __launch_bounds__(256) quant_act_weight_kernel(ActWeightArgs a) {
  __shared__ float wave_max[4];
  const int b = static_cast<int>(blockIdx.x);
  if (b < a.n_w)
    weight_block<WBF16, POW2>(b, a.w, a.ld_w, a.GK, a.q_w, a.s_w, a.K_w, wave_max);
  else
    act_rows_block<XBF16, POW2>(b - a.n_w, a.x, a.ld_x, a.G, a.tiles, a.q_x, a.s_x, a.K_x);
}

// 4 x 4 byte transpose: t[e] byte r = byte e of r4[r].
__device__ __forceinline__ void transpose4x4(const uint32_t (&r4)[4], uint32_t (&t)[4]) {
  const uint32_t x0 = __builtin_amdgcn_perm(r4[1], r4[0], 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t x1 = __builtin_amdgcn_perm(r4[1], r4[0], 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t y0 = __builtin_amdgcn_perm(r4[3], r4[2], 0x05010400u);
  const uint32_t y1 = __builtin_amdgcn_perm(r4[3], r4[2], 0x07030602u);
  t[0] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
  t[1] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
  t[2] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
  t[3] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
}

// 128x128 quantisation that writes the codes twice: row-major q [N,K] and
// transposed q_t [K,N].  The blocks of W^T are the transposes of the blocks of
// W with the same amax, so q_t and scales_t (= scales transposed) are exactly
// the 128x128 quantisation of W^T: the B operand of the data-gradient GEMM.
// Thread (q4, cg) holds rows 4*q4 .. 4*q4+3 of the block, 16 columns each in
// the run layout of the 1x128 quantiser (lane cg of 8: runs of L columns at
// r * 8L + cg * L), so every load instruction reads 128 contiguous bytes of a
// row (40.8 -> 35.5 us on [7168,7168] bf16 against 16 consecutive columns per
// thread).  It writes its codes as 4 x 4 blocks (rows 4*q4.., 4 consecutive
// columns; a 4x4 byte transpose) into an LDS tile of the transposed block,
// whose 32-dword rows c are XOR-permuted by ((c / L) & 3) << 3 (two lanes per
// bank at most), and the tile leaves as full 128-byte rows.
template <bool BF16, bool POW2>
__global__ void __launch_bounds__(256) quant_weight_dual_kernel(const void* __restrict__ w, int64_t ld, int GK, int GN,
                                                                uint8_t* __restrict__ q, float* __restrict__ scales,
                                                                uint8_t* __restrict__ qt, float* __restrict__ scales_t,
                                                                int64_t N, int64_t K) {
  __shared__ float wave_max[4];
  __shared__ __attribute__((aligned(16))) uint32_t tr[128 * 32];
  using R = Runs<BF16>;
  const int bi = blockIdx.x / GK;
  const int bj = blockIdx.x - bi * GK;
  const int cg = threadIdx.x & 7;
  const int q4 = threadIdx.x >> 3;
  float v[4][16];
  float amax = 0.0f;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t row = static_cast<int64_t>(bi) * 128 + 4 * q4 + rr;
    load_runs<BF16>(static_cast<const char*>(w) + (row * ld + static_cast<int64_t>(bj) * 128) * R::ES, cg, v[rr]);
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[rr][e]));
  amax = max64(amax);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  float s, inv;
  group_scale<POW2>(amax, s, inv);
  uint32_t codes[4][4];  // [row rr][dword d]: elements 4d .. 4d+3 of the thread's 16
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t row = static_cast<int64_t>(bi) * 128 + 4 * q4 + rr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      codes[rr][d] = cvt4(v[rr][4 * d] * inv, v[rr][4 * d + 1] * inv, v[rr][4 * d + 2] * inv, v[rr][4 * d + 3] * inv);
    store_runs<BF16>(u32x4{codes[rr][0], codes[rr][1], codes[rr][2], codes[rr][3]},
                     q + row * K + static_cast<int64_t>(bj) * 128, cg);
  }
  // Transposed tile: row c = column of the block (a K index), dword q4 = its 4
  // codes of rows 4*q4 .. 4*q4+3.  Code dword d of the thread covers columns
  // col(d / (L/4), cg) + 4 * (d % (L/4)) .. +3.
  constexpr int DPR = R::L / 4;  // code dwords per run
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t r4[4] = {codes[0][d], codes[1][d], codes[2][d], codes[3][d]};
    uint32_t t[4];
    transpose4x4(r4, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = R::col(d / DPR, cg) + 4 * (d % DPR) + e;
      tr[c * 32 + (q4 ^ (((c / R::L) & 3) << 3))] = t[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int idx = threadIdx.x + 256 * t;
    const int c = idx >> 3, ch = idx & 7;
    const u32x4 val = *reinterpret_cast<const u32x4*>(&tr[c * 32 + 4 * (ch ^ (((c / R::L) & 3) << 1))]);
    store_codes(val, reinterpret_cast<u32x4*>(qt + (static_cast<int64_t>(bj) * 128 + c) * N +
                                                              static_cast<int64_t>(bi) * 128 + ch * 16));
  }
  if (threadIdx.x == 0) {
    scales[blockIdx.x] = s;
    scales_t[static_cast<int64_t>(bj) * GN + bi] = s;
  }
}

}  // namespace

hipError_t launch_quant_act_rows(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, int64_t ld,
                                 uint8_t* q, float* scales, hipStream_t s) {
  const int G = static_cast<int>(K / 128);
  const int64_t tiles = M * G;
  const dim3 grid(static_cast<unsigned>((tiles + 31) / 32));
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, x, ld, G, tiles, q, scales, K); };
  if (bf16)
    pow2 ? go(quant_act_rows_kernel<true, true>) : go(quant_act_rows_kernel<true, false>);
  else
    pow2 ? go(quant_act_rows_kernel<false, true>) : go(quant_act_rows_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_quant_per_tensor(const void* x, bool bf16, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                                   float* scales, int64_t n_scales, hipStream_t s) {
  const int G = static_cast<int>(K / 128);
  const int64_t tiles = M * G;
  // (1) writes one partial per block into the scale slots, so at most n_scales
  // blocks (and at most 2048: each then strides over the tile grid)
  int64_t nb = (tiles + 31) / 32;
  nb = nb < n_scales ? nb : n_scales;
  nb = nb < 2048 ? nb : 2048;
  if (bf16)
    hipLaunchKernelGGL(quant_pt_amax_kernel<true>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, x, ld, G, tiles,
                       scales);
  else
    hipLaunchKernelGGL(quant_pt_amax_kernel<false>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, x, ld, G, tiles,
                       scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_pt_scale_kernel, dim3(1), dim3(256), 0, s, scales, static_cast<int>(nb));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((tiles + 31) / 32));
  if (bf16)
    hipLaunchKernelGGL(quant_pt_cast_kernel<true>, grid, dim3(256), 0, s, x, ld, G, tiles, q, scales, n_scales, K);
  else
    hipLaunchKernelGGL(quant_pt_cast_kernel<false>, grid, dim3(256), 0, s, x, ld, G, tiles, q, scales, n_scales, K);
  return hipGetLastError();
}

hipError_t launch_quant_act_cols(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, int64_t ld,
                                 uint8_t* q, float* scales, hipStream_t s) {
  const int G = static_cast<int>(K / 128);
  const int tile_cols = kColsTileBytes / (bf16 ? 2 : 4);
  const int CB = static_cast<int>((M + tile_cols - 1) / tile_cols);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(CB) * G));
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(512), 0, s, x, ld, M, G, CB, q, scales, K); };
  if (bf16)
    pow2 ? go(quant_act_cols_kernel<true, true>) : go(quant_act_cols_kernel<true, false>);
  else
    pow2 ? go(quant_act_cols_kernel<false, true>) : go(quant_act_cols_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, int64_t ld,
                               uint8_t* q, float* scales, hipStream_t s) {
  const int GK = static_cast<int>(K / 128);
  const dim3 grid(static_cast<unsigned>((N / 128) * GK));
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, w, ld, GK, q, scales, K); };
  if (bf16)
    pow2 ? go(quant_weight_kernel<true, true>) : go(quant_weight_kernel<true, false>);
  else
    pow2 ? go(quant_weight_kernel<false, true>) : go(quant_weight_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_quant_act_weight(const void* x, bool x_bf16, int64_t M, int64_t K_x, int64_t ld_x, uint8_t* q_x,
                                   float* s_x, const void* w, bool w_bf16, int64_t N, int64_t K_w, int64_t ld_w,
                                   uint8_t* q_w, float* s_w, bool pow2, hipStream_t s) {
  ActWeightArgs a{};
  a.x = x; a.ld_x = ld_x; a.K_x = K_x; a.G = static_cast<int>(K_x / 128); a.tiles = M * (K_x / 128);
  a.q_x = q_x; a.s_x = s_x;
  a.w = w; a.ld_w = ld_w; a.K_w = K_w; a.GK = static_cast<int>(K_w / 128);
  a.n_w = static_cast<int>((N / 128) * (K_w / 128));
  a.q_w = q_w; a.s_w = s_w;
  const int64_t n_x = (a.tiles + 31) / 32;
  const dim3 grid(static_cast<unsigned>(a.n_w + n_x));
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, a); };
  if (x_bf16 && w_bf16)
    pow2 ? go(quant_act_weight_kernel<true, true, true>) : go(quant_act_weight_kernel<true, true, false>);
  else if (x_bf16)
    pow2 ? go(quant_act_weight_kernel<true, false, true>) : go(quant_act_weight_kernel<true, false, false>);
  else if (w_bf16)
    pow2 ? go(quant_act_weight_kernel<false, true, true>) : go(quant_act_weight_kernel<false, true, false>);
  else
    pow2 ? go(quant_act_weight_kernel<false, false, true>) : go(quant_act_weight_kernel<false, false, false>);
  return hipGetLastError();
}

hipError_t launch_quant_weight_dual(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, int64_t ld,
                                    uint8_t* q, float* scales, uint8_t* qt, float* scales_t, hipStream_t s) {
  const int GK = static_cast<int>(K / 128), GN = static_cast<int>(N / 128);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(GN) * GK));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, w, ld, GK, GN, q, scales, qt, scales_t, N, K);
  };
  if (bf16)
    pow2 ? go(quant_weight_dual_kernel<true, true>) : go(quant_weight_dual_kernel<true, false>);
  else
    pow2 ? go(quant_weight_dual_kernel<false, true>) : go(quant_weight_dual_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace fp8fg
