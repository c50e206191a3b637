// Device code of fp8bq: blockwise BF16 -> OCP e4m3fn quantization for gfx950.
//
// The arithmetic is the blockwise cast of the page "fp8_kernel.py — FP8 量化内核"
// (section 2, Triton implementation): per tile, a = max(max|x|, eps),
// s = a/448 (stored), r = 1/s, q = e4m3fn(clamp(x*r, -448, 448)).
//
// Work decomposition (one 256-thread workgroup = 4 wave64s per work unit):
//   * every thread owns 16-byte column chunks (8 BF16 values) of a unit that
//     is 128 columns wide: 16 threads cover one 256-byte row segment, so a
//     wave's load touches 4 rows x 256 contiguous bytes and its 8-byte FP8
//     store writes 4 rows x 128 contiguous bytes (whole cache lines);
//   * [128,128] blocks: unit = one tile (8 loads per thread, all held in
//     registers: the tile is read from HBM exactly once), or, for launches
//     of wide and many tiles, four side-by-side tiles (128 x 512, 32 loads
//     per thread) so that every wave load reads one 1 KB row run;
//   * [64,64] blocks: unit = 64 x 128 = two side-by-side tiles, so the FP8
//     rows written are still full 128-byte lines, or, for launches of wide
//     and many tiles, eight side-by-side tiles (64 x 512, 16 loads per
//     thread, 1 KB row runs per wave load);
//   * [1,128] blocks: unit = 64 rows x 128 = 64 row-tiles; each tile's
//     maximum is reduced inside one 16-lane DPP row, with no LDS and no
//     barrier, and each lane divides for one row-tile only (DPP quad
//     broadcast of the reciprocals); when N % 128 == 0 the unit is instead
//     64 consecutive row-tiles of the flat array (16 KB contiguous), in
//     kernels of their own;
//   * any other block size (one tile per unit): up to 16384 elements with
//     8-aligned columns, the whole tile in registers; up to 65536, two
//     16-byte passes over the tile; N % 8 != 0 or a misaligned pointer,
//     element by element;
//   * one scale per tensor (a single tile of 2^20 or more values that fits
//     in the registers of the grid the chip holds at once, about 50 M
//     values): the tensor is read once and held in registers while the
//     workgroups agree on its maximum through device-scope atomics
//     (section "one scale per tensor, held in registers"), one launch per
//     tensor or one persistent launch per list;
//   * other tiles of more than 65536 elements and shards that start inside
//     a tile: two passes over chunks of each tile (section "large tiles"):
//     per-workgroup maxima in slots of q and a reduce kernel for whole
//     tensors, atomic maxima for shards;
//   * shards whose tiles hold at most 16384 elements with 8-aligned tile
//     columns: one workgroup per tile (64-row units for one-row tiles), the
//     maxima pass and the quantize pass each one launch, singly or grouped
//     (section "small tiles of shards").
// Every body computes the same arithmetic, so results never depend on it.
// The file also holds dequantization (decode(q) * s, section
// "dequantization", singly or over a list in one launch) and the final cast
// on its own.
//
// The tile maximum is an integer max over (bits & 0x7FFF): for finite BF16
// values magnitude order equals bit-pattern order, so this is exact.
//
// Every byte is touched once, so the vector bodies load and store with the
// nontemporal hint (streaming data that no later access reuses); together
// with the XCD-aware unit order below this lifts the measured rate of the
// grouped launch from about 67% to about 77% of the 8 TB/s HBM peak.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "div31.hpp"

namespace fp8bq {

constexpr float kE4m3Max = 448.0f;
constexpr float kEps = 1e-10f;
constexpr int kThreads = 256;

enum Kind : int { kT128 = 0, kT64 = 1, kR128 = 2, kGeneral = 3, kT128W = 4, kT64W = 5 };

// Pointers into device memory, marked as global so loads and stores are
// emitted as global_* (not flat_*) instructions.
#define FP8BQ_GLOBAL __attribute__((address_space(1)))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// One tensor as the kernels see it.
struct Desc {
  const uint16_t* x;  // BF16 [M, N]
  uint8_t* q;         // e4m3fn [M, N]
  float* s;           // fp32 [TM, TN]
  int64_t M;
  int64_t N;
  int32_t TN;       // tile columns: row pitch of s
  int32_t UN;       // work-unit columns
  int32_t body;     // which unit body this tensor takes (Body below)
  int32_t pad;
  int64_t reserved;  // pads the entry to 64 bytes
};

// Unit bodies: the block-shape kernel of the launch (a [128,128], [64,64] or
// [1,128] unit), a whole tile held in registers (any block of at most
// kRegTile elements with 8-aligned columns), a larger tile in two vector
// passes (8-aligned columns), a tile element by element, or (for [1,128]
// blocks with N % 128 == 0) 64 consecutive row-tiles of the flat array.
enum Body : int { kBodyVec = 0, kBodyScalar = 1, kBodyRegTile = 2, kBodyLoopVec = 3, kBodyFlat = 4 };
constexpr int64_t kRegTile = 16384;
static_assert(sizeof(Desc) == 64, "descriptor layout is part of the workspace format");

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a);
  u16x2 y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Packed magnitudes of the 8 BF16 values of a chunk, folded to two u16 maxima.
__device__ __forceinline__ uint32_t fold_abs(u32x4 w) {
  constexpr uint32_t kMag = 0x7FFF7FFFu;
  uint32_t a = pk_max_u16(w.x & kMag, w.y & kMag);
  uint32_t b = pk_max_u16(w.z & kMag, w.w & kMag);
  return pk_max_u16(a, b);
}

__device__ __forceinline__ uint32_t halves_max(uint32_t m) {
  return max(m & 0xFFFFu, m >> 16);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  int o = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return max(v, (uint32_t)o);
}

// Max over each aligned group of 8 lanes (quad swaps, then half-row mirror).
__device__ __forceinline__ uint32_t max8(uint32_t v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  return v;
}

// Max over each 16-lane DPP row.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  return dpp_max<0x140>(max8(v));  // row_mirror
}

// Max of lanes L, L+16, L+32, L+48 (one value per DPP row), as a uniform value.
template <int L>
__device__ __forceinline__ uint32_t rows_max(uint32_t v) {
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, L);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, L + 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, L + 32);
  uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, L + 48);
  return max(max(a, b), max(c, d));
}

// Compile-time loop: f(std::integral_constant<int, K>) for K = 0 .. N-1.
template <typename F, int... K>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value of lane K of each quad (4 consecutive lanes), for every lane of it.
template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), K | (K << 2) | (K << 4) | (K << 6), 0xF, 0xF, false));
}

// Scale and reciprocal from a tile's maximum magnitude: two correctly rounded
// binary32 divisions (this file is built without fast-math).
__device__ __forceinline__ void tile_scale_f(float amax, float& s, float& r) {
  const float a = fmaxf(amax, kEps);
  s = a / kE4m3Max;
  r = 1.0f / s;
}

// Same from the maximum's BF16 magnitude bits (widened exactly to fp32).
__device__ __forceinline__ void tile_scale(uint32_t maxbits, float& s, float& r) {
  tile_scale_f(__uint_as_float(maxbits << 16), s, r);
}

__device__ __forceinline__ float clamp448(float y) {
  return __builtin_amdgcn_fmed3f(y, -kE4m3Max, kE4m3Max);
}

// Four clamped values -> four e4m3fn bytes (byte i = value i).
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 BF16 values (one 16-byte chunk) -> 8 e4m3fn bytes.
__device__ __forceinline__ u32x2 quant8(u32x4 w, float r) {
  u32x2 o;
  o.x = cvt4(clamp448(bf_lo(w.x) * r), clamp448(bf_hi(w.x) * r),
             clamp448(bf_lo(w.y) * r), clamp448(bf_hi(w.y) * r));
  o.y = cvt4(clamp448(bf_lo(w.z) * r), clamp448(bf_hi(w.z) * r),
             clamp448(bf_lo(w.w) * r), clamp448(bf_hi(w.w) * r));
  return o;
}

// ---------------------------------------------------------------- unit bodies

template <int KIND>
struct UnitShape {
  static constexpr int kRows = (KIND == kT128) ? 128 : 64;  // unit rows
  static constexpr int kLoads = kRows / 16;                 // 16-byte loads per thread
};

// Vectorized unit (ur, uc) of a [128,128], [64,64] or [1,128] tensor.
// CHECK = the unit crosses the bottom or right edge of the matrix.
// Needs N % 8 == 0, x 16-byte and q 8-byte aligned.
template <int KIND, bool CHECK>
__device__ __forceinline__ void vec_unit(const Desc& d, int64_t ur, int64_t uc, uint32_t* red) {
  constexpr int R = UnitShape<KIND>::kRows;
  constexpr int L = UnitShape<KIND>::kLoads;
  const int t = threadIdx.x;
  const int chunk = t & 15;   // 16-byte column chunk within the unit
  const int prow = t >> 4;    // row within a 16-row pass
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t N = d.N;
  const int64_t row0 = ur * R;
  const int64_t col = uc * 128 + chunk * 8;
  int rows_valid = R;
  bool col_ok = true;
  if (CHECK) {
    const int64_t left = d.M - row0;
    rows_valid = left < R ? (int)left : R;
    col_ok = col < N;  // N % 8 == 0: a chunk is wholly inside or outside
  }
  const size_t base = (size_t)(row0 + prow) * (size_t)N + (size_t)col;
  const FP8BQ_GLOBAL u32x4* xp = (const FP8BQ_GLOBAL u32x4*)(d.x + base);
  const size_t pitch16 = (size_t)N * 16 / 8;  // 16 rows, in 16-byte chunks

  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    if (!CHECK || (col_ok && k * 16 + prow < rows_valid)) {
      v[k] = __builtin_nontemporal_load(&xp[k * pitch16]);
    } else {
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  FP8BQ_GLOBAL u32x2* qp = (FP8BQ_GLOBAL u32x2*)(d.q + base);
  FP8BQ_GLOBAL float* sp = (FP8BQ_GLOBAL float*)d.s;
  const size_t qpitch16 = (size_t)N * 16 / 8;  // 16 rows, in 8-byte chunks

  if constexpr (KIND == kR128) {
    // Every 16-lane DPP row holds one row-tile per load: reduce inside it.
    // A lane owns L = 4 row-tiles, so instead of 4 division pairs each lane
    // computes one -- for the row-tile k = chunk % 4 -- and the quad
    // (chunks 4j..4j+3) shares the four reciprocals by DPP broadcast.
    static_assert(L == 4, "one division per lane needs 4 row-tiles per lane");
    uint32_t m[L];
#pragma unroll
    for (int k = 0; k < L; ++k) m[k] = max16(halves_max(fold_abs(v[k])));
    const int mine = chunk & 3;
    const uint32_t msel = mine == 0 ? m[0] : mine == 1 ? m[1] : mine == 2 ? m[2] : m[3];
    float ssel, rsel;
    tile_scale(msel, ssel, rsel);
    static_for<L>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const float r = quad_bcast<k>(rsel);
      const bool row_ok = !CHECK || k * 16 + prow < rows_valid;
      if (row_ok && (!CHECK || col_ok)) __builtin_nontemporal_store(quant8(v[k], r), &qp[k * qpitch16]);
      if (chunk == k && row_ok) sp[(size_t)(row0 + k * 16 + prow) * d.TN + uc] = ssel;
    });
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < L; ++k) m = pk_max_u16(m, fold_abs(v[k]));
    m = halves_max(m);
    uint32_t tm;
    if constexpr (KIND == kT128) {
      m = max16(m);
      const uint32_t wm = rows_max<0>(m);
      if (lane == 0) red[wave] = wm;
      __syncthreads();
      tm = max(max(red[0], red[1]), max(red[2], red[3]));
    } else {  // kT64: left tile = chunks 0..7, right tile = chunks 8..15
      m = max8(m);
      const uint32_t w0 = rows_max<0>(m);
      const uint32_t w1 = rows_max<8>(m);
      if (lane == 0) {
        red[wave * 2] = w0;
        red[wave * 2 + 1] = w1;
      }
      __syncthreads();
      const int h = chunk >> 3;
      tm = max(max(red[h], red[2 + h]), max(red[4 + h], red[6 + h]));
    }
    float s, r;
    tile_scale(tm, s, r);
#pragma unroll
    for (int k = 0; k < L; ++k) {
      if (!CHECK || (col_ok && k * 16 + prow < rows_valid)) {
        __builtin_nontemporal_store(quant8(v[k], r), &qp[k * qpitch16]);
      }
    }
    if constexpr (KIND == kT128) {
      if (t == 0) sp[(size_t)ur * d.TN + uc] = s;
    } else {
      const int64_t tj = uc * 2 + (chunk >> 3);
      if ((t == 0 || t == 8) && tj < d.TN) sp[(size_t)ur * d.TN + tj] = s;
    }
  }
}

// [128,128] blocks, wide unit (kind kT128W): 128 rows x 512 columns, four
// side-by-side tiles per workgroup.  Lane c of a wave holds columns
// 8c..8c+7 of a 512-column row run (16-lane DPP row d = tile d of the
// unit), and wave w holds rows w, w+4, ..., w+124, so every wave load reads
// one contiguous 1 KB run and every store writes 512 contiguous bytes.  32
// loads per thread (all held in registers, about 224 VGPRs: 2 workgroups
// per CU).  A tile's maximum: fold over the thread's 32 loads, max over its
// DPP row, then over the 4 waves through LDS.  Against the one-tile unit
// this moved the 252-tensor dense set from 77.1% to 80.3% of the HBM peak
// (data-movement probes: 128x128 units 76.6-78.3%, 128x512 80.7%), but
// launches of few or half-empty units lose (one MoE layer: 76.3% -> 74.1%),
// so the host picks it per launch.  Also measured and not kept: two-tile
// 128x256 units (dense set 76.7%, below both), and MoE launches that give
// the 2048-wide matrices wide units and the 768-wide ones one-tile units
// (74.8% against 77.0% with one-tile units throughout), and eight-tile
// 128x1024 units on 512-thread workgroups (single calls on 151937x4096 and
// 32768x16384: 72-76% against 77-78%), and three-tile 128x384 units (48 of
// 64 lanes active) for the MoE layers' 768-wide matrices beside four-tile
// units for their 2048-wide ones (75.8% against 76.9%), and 256 x 256 units
// of two by two tiles (32 loads per thread, all lanes active: each wave load
// reads two 512-byte runs) for those 768-wide matrices beside four-tile
// units, both layouts in one body switched by a per-tensor flag (MoE layers
// 72.0% against 76.5%; the flag's extra arithmetic also cost the dense set
// 81.4% -> 79.2%), and raw buffer loads
// and stores for interior units, the row step in the scalar offset and no
// per-load address arithmetic (dense set 75.6-76.5% against 81.1%: the
// compiler's split of these global loads, 22 then 10, runs faster), and a
// raised wave priority (s_setprio 2) over the stores (no change) or over
// the loads (dense set +0.1%, 151937x4096 -1.1%).
template <bool CHECK>
__device__ __forceinline__ void vec_unit_wide(const Desc& d, int64_t ur, int64_t uc, uint32_t* red) {
  constexpr int L = 32;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int sub = lane >> 4;
  const int64_t N = d.N;
  const int64_t row0 = ur * 128;
  const int64_t col = uc * 512 + lane * 8;
  int rows_valid = 128;
  bool col_ok = true;
  if (CHECK) {
    const int64_t left = d.M - row0;
    rows_valid = left < 128 ? (int)left : 128;
    col_ok = col < N;  // N % 8 == 0: a chunk is wholly inside or outside
  }
  const size_t base = (size_t)(row0 + wave) * (size_t)N + (size_t)col;
  const FP8BQ_GLOBAL u32x4* xp = (const FP8BQ_GLOBAL u32x4*)(d.x + base);
  const size_t pitch16 = (size_t)N * 4 / 8;  // 4 rows, in 16-byte chunks
  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    if (!CHECK || (col_ok && k * 4 + wave < rows_valid)) {
      v[k] = __builtin_nontemporal_load(&xp[k * pitch16]);
    } else {
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < L; ++k) m = pk_max_u16(m, fold_abs(v[k]));
  m = max16(halves_max(m));
  if ((lane & 15) == 0) red[wave * 4 + sub] = m;
  __syncthreads();
  const uint32_t tm = max(max(red[sub], red[4 + sub]), max(red[8 + sub], red[12 + sub]));
  float s, r;
  tile_scale(tm, s, r);
  FP8BQ_GLOBAL u32x2* qp = (FP8BQ_GLOBAL u32x2*)(d.q + base);
  const size_t qpitch8 = (size_t)N * 4 / 8;  // 4 rows, in 8-byte chunks
#pragma unroll
  for (int k = 0; k < L; ++k) {
    if (!CHECK || (col_ok && k * 4 + wave < rows_valid)) {
      __builtin_nontemporal_store(quant8(v[k], r), &qp[k * qpitch8]);
    }
  }
  const int64_t tj = uc * 4 + sub;
  if (wave == 0 && (lane & 15) == 0 && (!CHECK || tj < d.TN)) {
    ((FP8BQ_GLOBAL float*)d.s)[(size_t)ur * d.TN + tj] = s;
  }
}

// [64,64] blocks, wide unit (kind kT64W): 64 rows x 512 columns, eight
// side-by-side tiles per workgroup, the [64,64] counterpart of the unit
// above.  Lane c holds columns 8c..8c+7 of a 512-column row run (8 lanes per
// tile: tile c / 8), wave w holds rows w, w+4, ..., w+60, so every wave load
// reads one contiguous 1 KB run.  16 loads per thread.  A tile's maximum:
// fold over the thread's loads, max over its 8 lanes, then over the 4 waves
// through LDS.  151937x4096: 79.0% -> 80.9% at 3 workgroups per CU, 82.4%
// at 2; the 252-tensor dense set at [64,64]: 79.4% -> 81.0% at 3 per CU
// (75.8% at 2).
template <bool CHECK>
__device__ __forceinline__ void vec_unit_wide64(const Desc& d, int64_t ur, int64_t uc, uint32_t* red) {
  constexpr int L = 16;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int sub = lane >> 3;
  const int64_t N = d.N;
  const int64_t row0 = ur * 64;
  const int64_t col = uc * 512 + lane * 8;
  int rows_valid = 64;
  if (CHECK) {
    const int64_t left = d.M - row0;
    rows_valid = left < 64 ? (int)left : 64;
  }
  const size_t base = (size_t)(row0 + wave) * (size_t)N + (size_t)col;
  const FP8BQ_GLOBAL u32x4* xp = (const FP8BQ_GLOBAL u32x4*)(d.x + base);
  const size_t pitch16 = (size_t)N * 4 / 8;
  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    if (!CHECK || 4 * k + wave < rows_valid) {
      v[k] = __builtin_nontemporal_load(&xp[k * pitch16]);
    } else {
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < L; ++k) m = pk_max_u16(m, fold_abs(v[k]));
  m = max8(halves_max(m));
  if ((lane & 7) == 0) red[wave * 8 + sub] = m;
  __syncthreads();
  const uint32_t tm = max(max(red[sub], red[8 + sub]), max(red[16 + sub], red[24 + sub]));
  float s, r;
  tile_scale(tm, s, r);
  FP8BQ_GLOBAL u32x2* qp = (FP8BQ_GLOBAL u32x2*)(d.q + base);
  const size_t qpitch8 = (size_t)N * 4 / 8;
#pragma unroll
  for (int k = 0; k < L; ++k) {
    if (!CHECK || 4 * k + wave < rows_valid) {
      __builtin_nontemporal_store(quant8(v[k], r), &qp[k * qpitch8]);
    }
  }
  if (wave == 0 && (lane & 7) == 0) {
    ((FP8BQ_GLOBAL float*)d.s)[(size_t)ur * d.TN + (size_t)uc * 8 + sub] = s;
  }
}

// A whole tile of at most kRegTile elements held in registers: rows x cols
// with cols % 8 == 0, x 16-byte and q 8-byte aligned, N % 8 == 0.  Vector v
// of the tile is row v / (cols/8), 8-column group v % (cols/8); thread t
// holds vectors t, t + 256, ... (at most 8), so the tile is read once.
__device__ __forceinline__ void reg_tile(const Desc& d, int32_t bm, int32_t bn, int64_t ti,
                                         int64_t tj, uint32_t* red) {
  const int t = threadIdx.x;
  const int64_t r0 = ti * bm;
  const int64_t c0 = tj * bn;
  const uint32_t rows = (uint32_t)((d.M - r0) < bm ? (d.M - r0) : bm);
  const uint32_t cols = (uint32_t)((d.N - c0) < bn ? (d.N - c0) : bn);
  const uint32_t vpr = cols / 8;
  const uint32_t nvec = rows * vpr;
  const size_t base = (size_t)r0 * d.N + c0;
  const FP8BQ_GLOBAL uint16_t* x = (const FP8BQ_GLOBAL uint16_t*)(d.x + base);
  FP8BQ_GLOBAL uint8_t* q = (FP8BQ_GLOBAL uint8_t*)(d.q + base);
  // A whole tile of exactly kRegTile elements whose 8-column groups per row
  // divide the workgroup: thread t holds row t / groups + k * (256 / groups),
  // one strided address per load and no per-load branch.
  const bool whole = nvec == (uint32_t)(kRegTile / 8) && (kThreads % vpr) == 0u;
  const uint32_t sh = whole ? (uint32_t)__builtin_ctz(vpr) : 0u;
  const size_t lane = (size_t)((uint32_t)t >> sh) * d.N + (size_t)((uint32_t)t & (vpr - 1u)) * 8;
  const size_t step = (size_t)(kThreads >> sh) * d.N;
  u32x4 v[8];
  size_t off[8];
  if (whole) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(x + lane + (size_t)k * step));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t vi = (uint32_t)t + (uint32_t)k * kThreads;
      if (vi < nvec) {
        const uint32_t rr = vi / vpr;
        off[k] = (size_t)rr * d.N + (size_t)(vi - rr * vpr) * 8;
        v[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(x + off[k]));
      } else {
        off[k] = 0;
        v[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = pk_max_u16(m, fold_abs(v[k]));
  m = max16(halves_max(m));
  const uint32_t wm = rows_max<0>(m);
  if ((t & 63) == 0) red[t >> 6] = wm;
  __syncthreads();
  const uint32_t tm = max(max(red[0], red[1]), max(red[2], red[3]));
  float s, r;
  tile_scale(tm, s, r);
  if (whole) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_nontemporal_store(quant8(v[k], r), (FP8BQ_GLOBAL u32x2*)(q + lane + (size_t)k * step));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t vi = (uint32_t)t + (uint32_t)k * kThreads;
      if (vi < nvec) __builtin_nontemporal_store(quant8(v[k], r), (FP8BQ_GLOBAL u32x2*)(q + off[k]));
    }
  }
  if (t == 0) ((FP8BQ_GLOBAL float*)d.s)[(size_t)ti * d.TN + tj] = s;
}

// Tile body for any block size and alignment: pass 1 takes the maximum,
// pass 2 re-reads the tile (mostly from cache) and writes it.  When the
// tile's columns are 8-aligned and the tensor is aligned (body kBodyLoopVec)
// both passes use 16-byte loads over vector v = (row v / (cols/8), 8-column
// group v % (cols/8)); otherwise they go element by element.  Tiles here
// hold at most kBigTile = 65536 elements (larger ones take the two-pass
// kernels), so in-tile indices use 32-bit arithmetic.
template <bool VEC>
__device__ __forceinline__ void general_tile(const Desc& d, int32_t bm, int32_t bn, int64_t ti,
                                             int64_t tj, uint32_t* red) {
  const uint32_t t = threadIdx.x;
  const int64_t r0 = ti * bm;
  const int64_t c0 = tj * bn;
  const uint32_t rows = (uint32_t)((d.M - r0) < bm ? (d.M - r0) : bm);
  const uint32_t cols = (uint32_t)((d.N - c0) < bn ? (d.N - c0) : bn);
  const uint32_t n = rows * cols;
  const FP8BQ_GLOBAL uint16_t* x = (const FP8BQ_GLOBAL uint16_t*)(d.x + (size_t)r0 * d.N + c0);
  FP8BQ_GLOBAL uint8_t* q = (FP8BQ_GLOBAL uint8_t*)(d.q + (size_t)r0 * d.N + c0);
  const uint32_t vpr = cols / 8;
  const uint32_t nvec = rows * vpr;
  uint32_t m = 0;
  if (VEC) {
    for (uint32_t v = t; v < nvec; v += kThreads) {
      const uint32_t rr = v / vpr;
      const u32x4 w = *(const FP8BQ_GLOBAL u32x4*)(x + (size_t)rr * d.N + (v - rr * vpr) * 8);
      m = max(m, halves_max(fold_abs(w)));
    }
  } else {
    for (uint32_t e = t; e < n; e += kThreads) {
      const uint32_t rr = e / cols;
      const uint32_t cc = e - rr * cols;
      m = max(m, (uint32_t)(x[(size_t)rr * d.N + cc] & 0x7FFFu));
    }
  }
  m = max16(m);
  const uint32_t wm = rows_max<0>(m);
  if ((t & 63) == 0) red[t >> 6] = wm;
  __syncthreads();
  const uint32_t tm = max(max(red[0], red[1]), max(red[2], red[3]));
  float s, r;
  tile_scale(tm, s, r);
  if (t == 0) ((FP8BQ_GLOBAL float*)d.s)[(size_t)ti * d.TN + tj] = s;
  if (VEC) {
    for (uint32_t v = t; v < nvec; v += kThreads) {
      const uint32_t rr = v / vpr;
      const size_t off = (size_t)rr * d.N + (v - rr * vpr) * 8;
      const u32x4 w = *(const FP8BQ_GLOBAL u32x4*)(x + off);
      __builtin_nontemporal_store(quant8(w, r), (FP8BQ_GLOBAL u32x2*)(q + off));
    }
  } else {
    for (uint32_t e = t; e < n; e += kThreads) {
      const uint32_t rr = e / cols;
      const uint32_t cc = e - rr * cols;
      const size_t off = (size_t)rr * d.N + cc;
      const float y = clamp448(__uint_as_float((uint32_t)x[off] << 16) * r);
      q[off] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFF);
    }
  }
}

// [1,128] blocks with N % 128 == 0: tile t is elements [128 t, 128 t + 128) of
// the flat array and its scale is scale_inv[t] (row-major [M, N/128]), so
// unit u is tiles 64u .. 64u + 63: 16 KB of contiguous BF16 in, 8 KB of
// codes and 256 B of scales out.  The lanes and the reduction are those of
// the [1,128] unit (16-lane DPP row = one tile; one division per lane, quad
// broadcast of the reciprocals).  Streaming 16 KB contiguous runs, at 4
// workgroups per CU, moves HBM faster than 64-row units of one tile column.
// TAIL: the unit holds the last tiles; lanes past them load and store
// nothing (full units have no branch around their loads).
template <bool TAIL>
__device__ __forceinline__ void flat_r128_unit(const Desc& d, int64_t u, int64_t ntiles) {
  const int t = threadIdx.x;
  const int chunk = t & 15;
  const int drow = t >> 4;
  const int64_t tile0 = u * 64 + drow;
  const FP8BQ_GLOBAL u32x4* xp = (const FP8BQ_GLOBAL u32x4*)(d.x + tile0 * 128 + chunk * 8);
  FP8BQ_GLOBAL u32x2* qp = (FP8BQ_GLOBAL u32x2*)(d.q + tile0 * 128 + chunk * 8);
  constexpr int64_t kStep = 16 * 128 / 8;  // 16 tiles, in 16-byte (and 8-byte) units
  u32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (!TAIL || tile0 + k * 16 < ntiles) {
      v[k] = __builtin_nontemporal_load(&xp[k * kStep]);
    } else {
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t m[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) m[k] = max16(halves_max(fold_abs(v[k])));
  const int mine = chunk & 3;
  const uint32_t msel = mine == 0 ? m[0] : mine == 1 ? m[1] : mine == 2 ? m[2] : m[3];
  float ssel, rsel;
  tile_scale(msel, ssel, rsel);
  static_for<4>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    const float r = quad_bcast<k>(rsel);
    if (!TAIL || tile0 + k * 16 < ntiles) __builtin_nontemporal_store(quant8(v[k], r), &qp[k * kStep]);
  });
  // lane `chunk` < 4 holds the scale of tile chunk*16 + drow of the unit
  const int64_t st = tile0 + mine * 16;
  if (chunk < 4 && (!TAIL || st < ntiles)) ((FP8BQ_GLOBAL float*)d.s)[st] = ssel;
}

__device__ __forceinline__ void flat_r128(const Desc& d, int64_t u) {
  const int64_t ntiles = d.M * (d.N / 128);
  if ((u + 1) * 64 <= ntiles) {
    flat_r128_unit<false>(d, u, ntiles);
  } else {
    flat_r128_unit<true>(d, u, ntiles);
  }
}

template <int KIND>
__device__ __forceinline__ void run_unit(const Desc& d, int32_t bm, int32_t bn, int64_t u,
                                         uint32_t* red) {
  if constexpr (KIND == kR128) {
    if (d.body == kBodyFlat) {
      flat_r128(d, u);
      return;
    }
  }
  // Units per tensor are < 2^31 (checked on the host): 32-bit division.
  const uint32_t uu = (uint32_t)u;
  const uint32_t un = (uint32_t)d.UN;
  const uint32_t ur = uu / un;
  const uint32_t uc = uu - ur * un;
  if constexpr (KIND == kGeneral) {
    // Register and loop-vector bodies need aligned tensors, which launches of
    // a vector kind always give the vector body: compile them here only.
    if (d.body == kBodyRegTile) {
      reg_tile(d, bm, bn, ur, uc, red);
    } else if (d.body == kBodyLoopVec) {
      general_tile<true>(d, bm, bn, ur, uc, red);
    } else {
      general_tile<false>(d, bm, bn, ur, uc, red);
    }
  } else if (d.body != kBodyVec) {
    general_tile<false>(d, bm, bn, ur, uc, red);
  } else if constexpr (KIND == kT64W) {
    // Whole 512-column units only (as for kT128W): the rows alone are tested.
    if ((int64_t)(ur + 1) * 64 <= d.M) {
      vec_unit_wide64<false>(d, ur, uc, red);
    } else {
      vec_unit_wide64<true>(d, ur, uc, red);
    }
  } else if constexpr (KIND == kT128W) {
    // The host picks this kind only for tensors whose width is a whole number
    // of 512-column units, so only the last unit row can be ragged.  Testing
    // the rows alone measured 1-2% faster than also testing the columns
    // (dense 36-layer set 80.1% -> 81.2% of peak, 151937x4096 78.9% -> 81.0%).
    const bool inside = (int64_t)(ur + 1) * 128 <= d.M;
    if (inside) {
      vec_unit_wide<false>(d, ur, uc, red);
    } else {
      vec_unit_wide<true>(d, ur, uc, red);
    }
  } else {
    constexpr int R = UnitShape<KIND>::kRows;
    const bool inside = (int64_t)(ur + 1) * R <= d.M && (int64_t)(uc + 1) * 128 <= d.N;
    if (inside) {
      vec_unit<KIND, false>(d, ur, uc, red);
    } else {
      vec_unit<KIND, true>(d, ur, uc, red);
    }
  }
}

// ---------------------------------------------------------------- kernels

// Workgroup -> work unit, XCD-aware.  Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs of the chip, each with its own L2.  Remapping
// so that XCD x handles the x-th contiguous eighth of the units keeps every
// XCD streaming one contiguous address range, which measurably raises the
// HBM rate of this read-2/write-1 stream (no unit is read twice either way).
// `n` units are spread over `n` workgroups; the map is a bijection on [0, n).
__device__ __forceinline__ int64_t xcd_unit(int64_t wg, int64_t n) {
  constexpr int64_t kXcds = 8;
  const int64_t per = n / kXcds;
  const int64_t rem = n % kXcds;
  const int64_t xcd = wg % kXcds;
  const int64_t idx = wg / kXcds;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Calls f(u) for the units this workgroup owns: units are handed out in
// rounds of gridDim.x (a dispatch holds at most 2^32 - 1 work-items, i.e.
// 16,777,215 workgroups of 256), XCD-aware within each round.  Barriers in f
// are safe: every thread of a workgroup runs the same rounds; a barrier
// between rounds lets f reuse its LDS scratch.
template <typename F>
__device__ __forceinline__ void for_each_unit(int64_t total, F&& f) {
  for (int64_t b0 = 0; b0 < total; b0 += gridDim.x) {
    const int64_t n = (total - b0) < (int64_t)gridDim.x ? (total - b0) : (int64_t)gridDim.x;
    if ((int64_t)blockIdx.x >= n) return;
    if (b0 > 0) __syncthreads();  // LDS scratch of the previous round is reused
    f(b0 + xcd_unit(blockIdx.x, n));
  }
}

// One tensor: workgroup -> unit -> (unit row, unit column) of d.  The grid
// normally equals `total`; larger counts are covered in grid-sized rounds.
template <int KIND>
__global__ __launch_bounds__(kThreads) void quantize_one(Desc d, int32_t bm, int32_t bn,
                                                         int64_t total) {
  __shared__ uint32_t red[32];
  for_each_unit(total, [&](int64_t u) {
    run_unit<KIND>(d, bm, bn, u, red);
  });
}

// One [1,128] tensor with N % 128 == 0 (flat units).  The same body runs
// inside quantize_one<kR128>, but a kernel of its own measured faster
// (151937x4096: 80.0-80.6% of peak inside, 82.4-83.4% alone).
__global__ __launch_bounds__(kThreads) void quantize_flat_one(Desc d, int64_t total) {
  for_each_unit(total, [&](int64_t u) { flat_r128(d, u); });
}

// Tensor that owns global unit u: the largest t < count with start[t] <= u
// (start[0] = 0 <= u, non-decreasing).  start is uniform, so the search runs
// on scalar loads.  For the quantize launches this beat counting the entries
// at or before u in one workgroup barrier (dense 36-layer set 81.0% against
// 73.4% of peak, MoE layers 76.7% against 74.4%), and the two-level search
// of the grouped dequantization (dense set 81.4% against 80.5%, MoE layers
// 77.5% against 76.4%, ragged set at [64,64] 79.4% against 73.8%): a
// quantize unit lives long enough to hide the search, and the extra scalar
// registers cost more than its latency.
template <typename T>
__device__ __forceinline__ int find_tensor(const T* start, int count, int64_t u) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= u) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  return lo;
}

// A list of tensors: start[t] is the first global unit of tensor t
// (start[0] = 0, strictly increasing: empty tensors are not listed).
template <int KIND>
__global__ __launch_bounds__(kThreads) void quantize_group(const Desc* __restrict__ descs,
                                                           const int64_t* __restrict__ start,
                                                           int32_t count, int32_t bm, int32_t bn,
                                                           int64_t total) {
  __shared__ uint32_t red[32];
  for_each_unit(total, [&](int64_t u) {
    const int lo = find_tensor(start, count, u);
    const Desc d = descs[lo];
    run_unit<KIND>(d, bm, bn, u - start[lo], red);
  });
}

// ---------------------------------------------------------------- large tiles and shards
//
// Tiles too large for one workgroup (per-tensor scales, [1, N] rows of
// huge N, any tile above kBigTile elements) and sub-matrices that start
// inside a tile (shards) take two passes over chunks of each tile.
//   Whole tensors: pass 1 stores one partial maximum per workgroup in its own
//   slot, kept in the q buffer that pass 2 overwrites later; a small kernel
//   reduces each tile's slots to its scale in scale_inv; pass 2 quantizes
//   with r = 1/s.  No atomics, three launches.
//   Shards (a sub-matrix whose element (0,0) sits at (row_phase, col_phase)
//   inside a tile of the full matrix's grid): pass 1 folds partial maxima
//   into the per-tile maxima with an atomic max (the caller combines shards'
//   maxima); pass 2 quantizes with given maxima and a last tiny kernel turns
//   maxima into scales.

constexpr int64_t kBigTile = 65536;     // elements; larger tiles take this path
constexpr int64_t kChunk = 16384;       // elements per workgroup pass

struct Big {
  const uint16_t* x;
  uint8_t* q;
  int64_t M;
  int64_t N;
  int32_t bm;
  int32_t bn;
  int32_t row_phase;
  int32_t col_phase;
  int64_t TMl;   // local tile rows
  int64_t TNl;   // local tile columns
  int64_t cpt;   // chunks per tile
  int64_t items; // TMl * TNl * cpt
  int32_t flat;  // tiles cover whole rows: a chunk is one contiguous range
  int32_t vec;   // x 16-byte aligned, q 8-byte aligned, N % 8 == 0
  int32_t cpm;   // chunks per pass-1 item, 1..kChunksPerMax
  int32_t pad;
};

// Rows [r0, r1) and columns [c0, c1) of local tile (ti, tj).
__device__ __forceinline__ void big_rect(const Big& b, int64_t ti, int64_t tj, int64_t& r0,
                                         int64_t& r1, int64_t& c0, int64_t& c1) {
  r0 = ti * b.bm - b.row_phase;
  r1 = r0 + b.bm;
  c0 = tj * b.bn - b.col_phase;
  c1 = c0 + b.bn;
  r0 = r0 < 0 ? 0 : r0;
  c0 = c0 < 0 ? 0 : c0;
  r1 = r1 > b.M ? b.M : r1;
  c1 = c1 > b.N ? b.N : c1;
}

// Workgroup-wide max of one value per thread (uniform result).
__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* red) {
  m = max16(m);
  const uint32_t wm = rows_max<0>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wm;
  __syncthreads();
  const uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();  // red[] is reused by the next call
  return r;
}

// One chunk of a large tile: PASS 0 returns this thread's max of the
// magnitude bits; PASS 1 quantizes the chunk with reciprocal r.
// Returns false when chunk k lies past the end of a short tile (uniform).
template <int PASS>
__device__ __forceinline__ bool big_chunk(const Big& b, int64_t tile, int64_t k, float r,
                                          uint32_t& m) {
  const int t = threadIdx.x;
  const FP8BQ_GLOBAL uint16_t* x = (const FP8BQ_GLOBAL uint16_t*)b.x;
  FP8BQ_GLOBAL uint8_t* q = (FP8BQ_GLOBAL uint8_t*)b.q;
  const int64_t ti = tile / b.TNl;
  const int64_t tj = tile - ti * b.TNl;
  int64_t r0, r1, c0, c1;
  big_rect(b, ti, tj, r0, r1, c0, c1);
  if (b.flat) {
    // The tile is rows [r0, r1) in full: one contiguous range of elements.
    const int64_t f0 = r0 * b.N + k * kChunk;
    int64_t f1 = f0 + kChunk;
    f1 = f1 > r1 * b.N ? r1 * b.N : f1;
    if (f0 >= f1) return false;
    int64_t head = f0;
    if (b.vec) {
      // f0 is a multiple of 8 (kChunk and N are), so 16-byte vectors from f0.
      const int64_t nv = (f1 - f0) / 8;
      const FP8BQ_GLOBAL u32x4* xv = (const FP8BQ_GLOBAL u32x4*)(x + f0);
      FP8BQ_GLOBAL u32x2* qv = (FP8BQ_GLOBAL u32x2*)(q + f0);
      constexpr int kPer = (int)(kChunk / 8 / kThreads);  // vectors per thread, full chunk
      if (nv == kChunk / 8) {
        u32x4 w[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) w[i] = __builtin_nontemporal_load(&xv[t + i * kThreads]);
        uint32_t mm = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (PASS == 0) {
            mm = pk_max_u16(mm, fold_abs(w[i]));
          } else {
            __builtin_nontemporal_store(quant8(w[i], r), &qv[t + i * kThreads]);
          }
        }
        if (PASS == 0) m = max(m, halves_max(mm));
      } else {
        for (int64_t v = t; v < nv; v += kThreads) {
          const u32x4 w = __builtin_nontemporal_load(&xv[v]);
          if (PASS == 0) {
            m = max(m, halves_max(fold_abs(w)));
          } else {
            __builtin_nontemporal_store(quant8(w, r), &qv[v]);
          }
        }
      }
      head = f0 + nv * 8;
    }
    for (int64_t e = head + t; e < f1; e += kThreads) {
      const uint32_t bits = x[e];
      if (PASS == 0) {
        m = max(m, bits & 0x7FFFu);
      } else {
        const float y = clamp448(__uint_as_float(bits << 16) * r);
        q[e] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFF);
      }
    }
    return true;
  }
  // General rectangle: rows of the chunk, element by element.
  const int64_t cols = c1 - c0;
  const int64_t rows_per = cols >= kChunk ? 1 : kChunk / cols;
  const int64_t ra = r0 + k * rows_per;
  int64_t rb = ra + rows_per;
  rb = rb > r1 ? r1 : rb;
  if (ra >= rb) return false;
  const int64_t n = (rb - ra) * cols;
  for (int64_t e = t; e < n; e += kThreads) {
    const int64_t rr = e / cols;
    const int64_t cc = e - rr * cols;
    const size_t off = (size_t)(ra + rr) * b.N + c0 + cc;
    const uint32_t bits = x[off];
    if (PASS == 0) {
      m = max(m, bits & 0x7FFFu);
    } else {
      const float y = clamp448(__uint_as_float(bits << 16) * r);
      q[off] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFF);
    }
  }
  return true;
}

// Pass 1 of the large-tile path.  Item `it` reduces b.cpm chunks of one
// tile (item it = tile * groups + g, groups = ceil(cpt / cpm)); the host
// picks b.cpm per tensor so that small tensors still spread over the chip.
//   SLOTS: the item's maximum magnitude bits go to out[it]: every item
//     writes its slot (0 for chunks past a short tile's end).
//   atomic: the maximum, as the fp32 bit pattern of the BF16 magnitude, is
//     folded into out[tile] (which must start at zero) with an atomic max,
//     skipped when a coherent read already shows a value at least as large.
//     Many workgroups folding into one address serialize on it, which is
//     why whole tensors take the slots.
constexpr int64_t kChunksPerMax = 16;       // largest b.cpm
constexpr int64_t kMaxItemsTarget = 2048;   // pass-1 items a tensor aims for (8 per CU)
constexpr int64_t kAtomicItemsTarget = 256; // the same with atomic maxima (1 per CU):
                                            // fewer workgroups folding into one address

// Pass-1 slots of a whole tensor: the first 4-byte-aligned address of q.
__host__ __device__ inline uint32_t* big_slots(uint8_t* q) {
  return reinterpret_cast<uint32_t*>((reinterpret_cast<uintptr_t>(q) + 3) & ~uintptr_t(3));
}

template <bool SLOTS>
__device__ __forceinline__ void big_max_item(const Big& b, uint32_t* out, int64_t it,
                                             uint32_t* red) {
  const int64_t cpm = b.cpm;
  const int64_t groups = (b.cpt + cpm - 1) / cpm;
  const int64_t tile = it / groups;
  const int64_t g = it - tile * groups;
  uint32_t m = 0;
  for (int64_t k = g * cpm; k < (g + 1) * cpm && k < b.cpt; ++k) {
    if (!big_chunk<0>(b, tile, k, 0.0f, m)) break;
  }
  const uint32_t wm = block_max(m, red);
  if (threadIdx.x != 0) return;
  if constexpr (SLOTS) {
    ((FP8BQ_GLOBAL uint32_t*)out)[it] = wm;
  } else if (wm != 0) {
    const uint32_t cur = __hip_atomic_load(&out[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((wm << 16) > cur) atomicMax(&out[tile], wm << 16);
  }
}

// Scale of one tile from its `groups` pass-1 slots: s = fl32(max(amax, eps) / 448).
__device__ __forceinline__ void big_reduce_tile(const uint32_t* slots, int64_t groups,
                                                int64_t tile, float* scale, uint32_t* red) {
  const FP8BQ_GLOBAL uint32_t* p = (const FP8BQ_GLOBAL uint32_t*)slots + tile * groups;
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < groups; i += kThreads) m = max(m, p[i]);
  m = block_max(m, red);
  if (threadIdx.x == 0) {
    float s, r;
    tile_scale(m, s, r);
    ((FP8BQ_GLOBAL float*)scale)[tile] = s;
  }
}

// Item `it` of pass 2 for one tensor: one chunk, quantized with its tile's
// scale (FROM_S: v holds s, and r = 1/s) or maximum (v holds amax, and s and
// r follow from it).  Both give the same r for the same tile.
template <bool FROM_S>
__device__ __forceinline__ void big_quant_item(const Big& b, const float* v, int64_t it) {
  const int64_t tile = it / b.cpt;
  const int64_t k = it - tile * b.cpt;
  const float vt = ((const FP8BQ_GLOBAL float*)v)[tile];
  float s, r;
  if constexpr (FROM_S) {
    s = vt;
    r = 1.0f / s;
  } else {
    tile_scale_f(vt, s, r);
  }
  uint32_t unused = 0;
  big_chunk<1>(b, tile, k, r, unused);
}

template <bool SLOTS>
__global__ __launch_bounds__(kThreads) void big_max(Big b, uint32_t* __restrict__ out,
                                                    int64_t items) {
  __shared__ uint32_t red[4];
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) big_max_item<SLOTS>(b, out, it, red);
}

// Tile scales of one whole tensor from its pass-1 slots.
__global__ __launch_bounds__(kThreads) void big_reduce(const uint32_t* __restrict__ slots,
                                                       int64_t groups, float* __restrict__ scale,
                                                       int64_t tiles) {
  __shared__ uint32_t red[4];
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) big_reduce_tile(slots, groups, t, scale, red);
}

template <bool FROM_S>
__global__ __launch_bounds__(kThreads) void big_quant(Big b, const float* __restrict__ v) {
  for (int64_t it = blockIdx.x; it < b.items; it += gridDim.x) big_quant_item<FROM_S>(b, v, it);
}

// Grouped form for a list of whole tensors with large tiles (phase 0): the
// table rides in the kernel arguments and each kernel covers every tensor,
// so a group costs 3 launches instead of 3 per tensor.
struct BigEntry {
  const uint16_t* x;
  uint8_t* q;
  float* s;        // scale_inv
  int32_t M;
  int32_t N;
  int32_t cpt;     // chunks per tile
  int32_t flags;   // bit 0: flat, bit 1: vec
  int32_t cpm;     // chunks per pass-1 item
  int32_t pad;
};

template <int CAP>
struct BigGroupArgs {
  int32_t tile_start[CAP + 1];   // prefix of tiles (reduce)
  int32_t max_start[CAP + 1];    // prefix of pass-1 items
  int32_t quant_start[CAP + 1];  // prefix of pass-2 items
  BigEntry e[CAP];
};

__device__ __forceinline__ Big big_of(const BigEntry& e, int32_t bm, int32_t bn) {
  Big b;
  b.x = e.x;
  b.q = e.q;
  b.M = e.M;
  b.N = e.N;
  b.bm = bm;
  b.bn = bn;
  b.row_phase = 0;
  b.col_phase = 0;
  b.TMl = ((int64_t)e.M + bm - 1) / bm;
  b.TNl = ((int64_t)e.N + bn - 1) / bn;
  b.cpt = e.cpt;
  b.items = b.TMl * b.TNl * b.cpt;
  b.flat = e.flags & 1;
  b.vec = (e.flags >> 1) & 1;
  b.cpm = e.cpm;
  b.pad = 0;
  return b;
}

template <int CAP>
__global__ __launch_bounds__(kThreads) void big_group_max(const BigGroupArgs<CAP> a, int32_t count,
                                                          int32_t bm, int32_t bn) {
  __shared__ uint32_t red[4];
  for_each_unit(a.max_start[count], [&](int64_t u) {
    const int t = find_tensor(a.max_start, count, u);
    const Big b = big_of(a.e[t], bm, bn);
    big_max_item<true>(b, big_slots(a.e[t].q), u - a.max_start[t], red);
  });
}

template <int CAP>
__global__ __launch_bounds__(kThreads) void big_group_reduce(const BigGroupArgs<CAP> a,
                                                             int32_t count) {
  __shared__ uint32_t red[4];
  for_each_unit(a.tile_start[count], [&](int64_t u) {
    const int t = find_tensor(a.tile_start, count, u);
    const BigEntry& e = a.e[t];
    const int64_t groups = ((int64_t)e.cpt + e.cpm - 1) / e.cpm;
    big_reduce_tile(big_slots(e.q), groups, u - a.tile_start[t], e.s, red);
  });
}

template <int CAP>
__global__ __launch_bounds__(kThreads) void big_group_quant(const BigGroupArgs<CAP> a, int32_t count,
                                                            int32_t bm, int32_t bn) {
  for_each_unit(a.quant_start[count], [&](int64_t u) {
    const int t = find_tensor(a.quant_start, count, u);
    const Big b = big_of(a.e[t], bm, bn);
    big_quant_item<true>(b, a.e[t].s, u - a.quant_start[t]);
  });
}

// out[i] = 0 for i < n.
// ---------------------------------------------------------------- one scale per tensor, held in registers
//
// A whole tensor with a single tile (one scale) that fits in the registers
// of one grid is read from HBM once instead of twice: every thread loads its
// share (up to kResMaxLoads 16-byte chunks, 8 values each) into registers,
// the workgroups combine their maxima, and each then quantizes the values it
// still holds.  3 bytes move per value instead of the two-pass path's 5.
//
// Cross-workgroup handshake, all through relaxed device-scope atomics (the
// only data that crosses workgroups is the atomics' own values):
//   * before the launch, resident_prep zeroes a count (q bytes 0..3) and a
//     maximum (q bytes 128..131, its own cache line: a shared line measured
//     15-20% slower) and writes kResNoScale into scale_inv (no scale is NaN);
//   * a workgroup raises the maximum, and only once that atomic has returned
//     increments the count (the count's operand depends on the returned
//     value); the workgroup that brings the count to the grid size reads the
//     maximum, computes the scale and stores it to scale_inv;
//   * the others poll scale_inv.  One that has waited longer than
//     `wait_ticks` (s_memrealtime ticks; the workgroups of a launch need not
//     all be resident at once, e.g. beside another launch) computes the
//     tensor's maximum itself from x: the scale is the same either way and
//     no wait is unbounded;
//   * only the last workgroup to arrive, which comes after every handshake
//     atomic, writes the codes of the two q chunks that hold the words
//     (loading those 16 values of x itself), with atomic exchanges in the
//     same coherence order; a workgroup past its wait limit may run ahead of
//     late arrivals, so no other workgroup writes there.
// Acquire/release ordering would make every workgroup write back and
// invalidate its L2 (measured: a fixed ~15 us per launch), and nothing but
// the atomics' values needs ordering.
//
// Loads and stores go through raw buffer resources sized to the tensor, with
// the whole byte offset in the per-lane (range-checked) offset: loads past
// the end return 0 (no effect on a maximum of magnitudes) and stores past
// the end are dropped, so the body has no bounds branches.

constexpr int kResMaxLoads = 48;            // chunks per thread, largest variant
constexpr uint32_t kResNoScale = 0xFFFFFFFFu;
constexpr int kResCountWord = 0;            // 32-bit word of q
constexpr int kResMaxWord = 32;             // 32-bit word of q (byte 128)
constexpr int kRawBufferFlags = 0x00020000; // buffer resource word 3: 32-bit format
constexpr int kNtPolicy = 2;                // nontemporal cache policy of buffer ops
constexpr uint32_t kResDropOffset = 0x7FFFFFF8u;  // past any tensor here: the store is dropped

struct ResTensor {
  uint8_t* q;
  float* s;
};

template <int CAP>
struct ResPrepArgs {
  ResTensor t[CAP];
};

template <int CAP>
__global__ void resident_prep(const ResPrepArgs<CAP> a, int32_t count) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= count) return;
  uint32_t* w = reinterpret_cast<uint32_t*>(a.t[i].q);
  w[kResCountWord] = 0u;
  w[kResMaxWord] = 0u;
  *reinterpret_cast<uint32_t*>(a.t[i].s) = kResNoScale;
}

// Thread 0 of a workgroup: contributes `bmax` and returns the scale's bits,
// or kResNoScale when the wait limit passed first.
__device__ __forceinline__ uint32_t resident_arrive(const uint16_t* x, uint32_t bmax, uint8_t* q,
                                                    float* s, uint32_t grid, uint64_t wait_ticks) {
  uint32_t* w = reinterpret_cast<uint32_t*>(q);
  uint32_t* sb = reinterpret_cast<uint32_t*>(s);
  const uint32_t prev =
      __hip_atomic_fetch_max(&w[kResMaxWord], bmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // prev <= 0x7FFF, so the operand is 1; the dependency orders the two atomics.
  const uint32_t old = __hip_atomic_fetch_add(&w[kResCountWord], 1u + (prev >> 31),
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old == grid - 1) {
    const uint32_t amax = __hip_atomic_load(&w[kResMaxWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float sf, rf;
    tile_scale(amax, sf, rf);
    const uint32_t sv = __float_as_uint(sf);
    __hip_atomic_store(sb, sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Every workgroup has arrived: the codes of the two handshake chunks.
    for (int c : {kResCountWord / 2, kResMaxWord / 2}) {
      const u32x2 o = quant8(*reinterpret_cast<const u32x4*>(x + c * 8), rf);
      __hip_atomic_exchange(reinterpret_cast<uint64_t*>(q + c * 8), (uint64_t)o.x | ((uint64_t)o.y << 32),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return sv;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t sv = __hip_atomic_load(sb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sv != kResNoScale) return sv;
    if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) return kResNoScale;
    __builtin_amdgcn_s_sleep(2);
  }
}

// The scale's bits from all of x, by one workgroup (the wait-limit path).
__device__ __forceinline__ uint32_t resident_scan(__amdgpu_buffer_rsrc_t xr, uint32_t nchunks,
                                                  uint32_t* red) {
  const uint32_t t = threadIdx.x;
  uint32_t m = 0;
  for (uint32_t c = t; c < nchunks; c += kThreads) {
    const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(c * 16u), 0, 0));
    m = pk_max_u16(m, fold_abs(w));
  }
  m = rows_max<0>(max16(halves_max(m)));
  __syncthreads();  // red[] may still be read by other waves
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  float sf, rf;
  tile_scale(max(max(red[0], red[1]), max(red[2], red[3])), sf, rf);
  return __float_as_uint(sf);
}

// One tensor of nchunks 16-byte chunks on `grid` workgroups, this one being
// number b (nchunks <= grid * kThreads * L, (nchunks + grid * kThreads * L)
// * 16 < 2^31, nchunks > kResMaxWord / 2).  Thread t holds chunks
// c0 + k * grid * kThreads, c0 = b * kThreads + t, so each wave load reads
// 1 KB contiguous.
template <int L>
__device__ __forceinline__ void resident_body(const uint16_t* __restrict__ x, uint8_t* q, float* s,
                                              uint32_t nchunks, uint32_t grid, uint32_t b,
                                              uint64_t wait_ticks, uint32_t* red) {
  const uint32_t t = threadIdx.x;
  const uint32_t stride = grid * kThreads;
  const uint32_t c0 = b * kThreads + t;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, (int)(nchunks * 16u), kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)(nchunks * 8u), kRawBufferFlags);
  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         xr, (int)((c0 + (uint32_t)k * stride) * 16u), 0, kNtPolicy));
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < L; ++k) m = pk_max_u16(m, fold_abs(v[k]));
  m = rows_max<0>(max16(halves_max(m)));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    red[4] = resident_arrive(x, max(max(red[0], red[1]), max(red[2], red[3])), q, s, grid, wait_ticks);
  }
  __syncthreads();
  uint32_t sv = red[4];
  if (sv == kResNoScale) sv = resident_scan(xr, nchunks, red);
  const float r = 1.0f / __uint_as_float(sv);
  // Chunks 0 and 16 hold the handshake words, which the last workgroup to
  // arrive writes: workgroup 0's stores there get an offset past the end,
  // which drops them.
  const bool word = b == 0 && (t == kResCountWord / 2 || t == kResMaxWord / 2);
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const u32x2 o = quant8(v[k], r);
    const uint32_t off = (k == 0 && word) ? kResDropOffset : (c0 + (uint32_t)k * stride) * 8u;
    __builtin_amdgcn_raw_buffer_store_b64(o, qr, (int)off, 0, kNtPolicy);
  }
}

template <int L>
__global__ __launch_bounds__(kThreads, 2) void resident_quant(const uint16_t* __restrict__ x,
                                                              uint8_t* q, float* s,
                                                              uint32_t nchunks,
                                                              uint64_t wait_ticks) {
  __shared__ uint32_t red[8];
  resident_body<L>(x, q, s, nchunks, gridDim.x, blockIdx.x, wait_ticks, red);
}

// A list of such tensors in one persistent launch: tensor i runs on the
// `grid` workgroups first, first + 1, ... (mod gridDim.x), and every
// workgroup takes its tensors in list order, so tensors on disjoint
// workgroups run side by side and no workgroup waits at a kernel boundary.
// A workgroup only ever waits for workgroups of the same tensor, which are
// at that tensor or at an earlier one, so the waits always end when the
// launch's workgroups are resident together (and the wait limit covers the
// case where they are not).
struct ResEntry {
  const uint16_t* x;
  uint8_t* q;
  float* s;
  uint32_t nchunks;
  uint32_t grid;
  uint32_t first;
  int32_t loads;  // L: 4, 8, 16, 32 or kResMaxLoads
};

template <int CAP>
struct ResGroupArgs {
  ResEntry e[CAP];
};

template <int CAP>
__global__ __launch_bounds__(kThreads, 2) void resident_group(const ResGroupArgs<CAP> a,
                                                              int32_t count,
                                                              uint64_t wait_ticks) {
  __shared__ uint32_t red[8];
  for (int32_t i = 0; i < count; ++i) {
    const ResEntry& e = a.e[i];
    const uint32_t b = blockIdx.x >= e.first ? blockIdx.x - e.first : blockIdx.x + gridDim.x - e.first;
    if (b >= e.grid) continue;
    __syncthreads();  // red[] of the previous tensor is no longer read
    switch (e.loads) {
      case 4: resident_body<4>(e.x, e.q, e.s, e.nchunks, e.grid, b, wait_ticks, red); break;
      case 8: resident_body<8>(e.x, e.q, e.s, e.nchunks, e.grid, b, wait_ticks, red); break;
      case 16: resident_body<16>(e.x, e.q, e.s, e.nchunks, e.grid, b, wait_ticks, red); break;
      case 32: resident_body<32>(e.x, e.q, e.s, e.nchunks, e.grid, b, wait_ticks, red); break;
      default: resident_body<kResMaxLoads>(e.x, e.q, e.s, e.nchunks, e.grid, b, wait_ticks, red); break;
    }
  }
}

// ---------------------------------------------------------------- small tiles of shards
//
// Shards whose tiles hold at most kRegTile elements, with tile columns that
// start on 8-element boundaries inside the shard (x 16-byte and q 8-byte
// aligned; N, bn and col_phase multiples of 8).  One workgroup owns one
// local tile, so pass 1 stores the tile's maximum directly (no atomics, no
// zero fill) and pass 2 quantizes with the given maximum and stores the
// scale (no finalize launch).  The tile's part inside the shard sits in
// registers, 16-byte vector v = (row v / (cols/8), 8-column group v % (cols/8)),
// as in reg_tile.

// PASS 0: out[tile] = max |x| over the tile's part (fp32 of the BF16
// magnitude).  PASS 1: quantize with a = amax[tile], out[tile] = s.  `amax`
// may be `out` itself: every thread takes a from LDS after a barrier, so the
// tile's entry is read before thread 0 overwrites it.
// The tile's values v[0..7] are loaded; off(k) is vector k's element offset
// from the tile's origin and valid(k) says whether it lies in the tile.
template <int PASS, typename Off, typename Valid>
__device__ __forceinline__ void shard_tile_finish(const Big& b, int64_t tile, size_t base,
                                                  const u32x4 (&v)[8], Off off, Valid valid,
                                                  float* out, uint32_t* red) {
  const int t = threadIdx.x;
  if (PASS == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = pk_max_u16(m, fold_abs(v[k]));
    m = max16(halves_max(m));
    const uint32_t wm = rows_max<0>(m);
    if ((t & 63) == 0) red[t >> 6] = wm;
    __syncthreads();
    const uint32_t tm = max(max(red[0], red[1]), max(red[2], red[3]));
    if (t == 0) ((FP8BQ_GLOBAL float*)out)[tile] = __uint_as_float(tm << 16);
  } else {
    __syncthreads();
    float sc, r;
    tile_scale_f(__uint_as_float(red[4]), sc, r);
    FP8BQ_GLOBAL uint8_t* q = (FP8BQ_GLOBAL uint8_t*)(b.q + base);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (valid(k)) __builtin_nontemporal_store(quant8(v[k], r), (FP8BQ_GLOBAL u32x2*)(q + off(k)));
    }
    if (t == 0) ((FP8BQ_GLOBAL float*)out)[tile] = sc;
  }
}

// PASS 0: out[tile] = max |x| over the tile's part (fp32 of the BF16
// magnitude).  PASS 1: quantize with a = amax[tile], out[tile] = s.  `amax`
// may be `out` itself: every thread takes a from LDS after a barrier, so the
// tile's entry is read before thread 0 overwrites it.  A whole tile of
// exactly kRegTile elements whose 8-column groups per row divide the
// workgroup (every interior [128,128] tile) takes a branch-free body: thread
// t holds row t / groups + k * (256 / groups), one strided address per load
// (151937x4096 shard at phase (64, 0): maxima pass 86.3% -> 89.3% of peak,
// quantize pass 72.3% -> 77.4%).
template <int PASS>
__device__ __forceinline__ void shard_small_tile(const Big& b, int64_t tile, const float* amax,
                                                 float* out, uint32_t* red) {
  const int t = threadIdx.x;
  const int64_t ti = tile / b.TNl;
  const int64_t tj = tile - ti * b.TNl;
  int64_t r0, r1, c0, c1;
  big_rect(b, ti, tj, r0, r1, c0, c1);
  const uint32_t vpr = (uint32_t)(c1 - c0) / 8;
  const uint32_t nvec = (uint32_t)(r1 - r0) * vpr;  // <= kRegTile / 8 = 8 per thread
  const size_t base = (size_t)r0 * b.N + c0;
  const FP8BQ_GLOBAL uint16_t* x = (const FP8BQ_GLOBAL uint16_t*)(b.x + base);
  if (PASS == 1) {
    if (t == 0) red[4] = __float_as_uint(((const FP8BQ_GLOBAL float*)amax)[tile]);
  }
  u32x4 v[8];
  if (nvec == (uint32_t)(kRegTile / 8) && (kThreads % vpr) == 0u) {
    const uint32_t sh = (uint32_t)__builtin_ctz(vpr);
    const size_t lane = (size_t)((uint32_t)t >> sh) * b.N + (size_t)((uint32_t)t & (vpr - 1u)) * 8;
    const size_t step = (size_t)(kThreads >> sh) * b.N;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(x + lane + (size_t)k * step));
    }
    shard_tile_finish<PASS>(b, tile, base, v, [&](int k) { return lane + (size_t)k * step; },
                            [](int) { return true; }, out, red);
    return;
  }
  size_t off[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t vi = (uint32_t)t + (uint32_t)k * kThreads;
    if (vi < nvec) {
      const uint32_t rr = vi / vpr;
      off[k] = (size_t)rr * b.N + (size_t)(vi - rr * vpr) * 8;
      v[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(x + off[k]));
    } else {
      off[k] = 0;
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  shard_tile_finish<PASS>(b, tile, base, v, [&](int k) { return off[k]; },
                          [&](int k) { return (uint32_t)t + (uint32_t)k * kThreads < nvec; }, out, red);
}

// Shards with one-row tiles of at most 128 columns ([1, bn], bn <= 128 and a
// multiple of 8; the row phase is then 0): a workgroup takes 64 rows of one
// tile column, as the [1,128] unit does.  Lane `c` of each 16-lane DPP row
// holds columns 8c..8c+7 of the tile, so a row-tile's maximum is reduced
// inside its DPP row; in pass 2 each lane computes the scale of one of its 4
// row-tiles and the quad shares the reciprocals.  A row-tile's given maximum
// is read by the lanes of its quad before the one lane that writes its
// scale does, so `amax` may be `out`.
template <int PASS>
__device__ __forceinline__ void shard_rows_unit(const Big& b, int64_t u, const float* amax,
                                                float* out) {
  const int t = threadIdx.x;
  const int chunk = t & 15;
  const int prow = t >> 4;
  const int64_t rb = u / b.TNl;
  const int64_t tj = u - rb * b.TNl;
  int64_t c0 = tj * b.bn - b.col_phase;
  int64_t c1 = c0 + b.bn;
  c0 = c0 < 0 ? 0 : c0;
  c1 = c1 > b.N ? b.N : c1;
  const int64_t col = c0 + chunk * 8;
  const bool col_ok = col < c1;
  const int64_t row0 = rb * 64 + prow;
  u32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t row = row0 + k * 16;
    v[k] = (col_ok && row < b.M)
               ? __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(b.x + row * b.N + col))
               : u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (PASS == 0) {
    static_for<4>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const uint32_t m = max16(halves_max(fold_abs(v[k])));
      const int64_t row = row0 + k * 16;
      if (chunk == 0 && row < b.M) ((FP8BQ_GLOBAL float*)out)[row * b.TNl + tj] = __uint_as_float(m << 16);
    });
  } else {
    const int mine = chunk & 3;
    const int64_t rm = row0 + mine * 16;
    const float a = rm < b.M ? ((const FP8BQ_GLOBAL float*)amax)[rm * b.TNl + tj] : 0.0f;
    float ssel, rsel;
    tile_scale_f(a, ssel, rsel);
    static_for<4>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const float r = quad_bcast<k>(rsel);
      const int64_t row = row0 + k * 16;
      if (col_ok && row < b.M) {
        __builtin_nontemporal_store(quant8(v[k], r), (FP8BQ_GLOBAL u32x2*)(b.q + row * b.N + col));
      }
    });
    if (chunk < 4 && rm < b.M) ((FP8BQ_GLOBAL float*)out)[rm * b.TNl + tj] = ssel;
  }
}

template <int PASS>
__global__ __launch_bounds__(kThreads) void shard_rows(Big b, const float* amax, float* out,
                                                       int64_t units) {
  for_each_unit(units, [&](int64_t u) { shard_rows_unit<PASS>(b, u, amax, out); });
}

template <int PASS>
__global__ __launch_bounds__(kThreads) void shard_small(Big b, const float* amax, float* out,
                                                        int64_t tiles) {
  __shared__ uint32_t red[32];
  for_each_unit(tiles, [&](int64_t tile) { shard_small_tile<PASS>(b, tile, amax, out, red); });
}

__global__ __launch_bounds__(kThreads) void fill_zero(uint32_t* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    ((FP8BQ_GLOBAL uint32_t*)out)[i] = 0u;
  }
}

// scale[i] = fl32(max(amax[i], eps) / 448); amax and scale may be the same array.
__global__ __launch_bounds__(kThreads) void finalize_scales(const float* amax, float* scale,
                                                            int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float s, r;
    tile_scale_f(((const FP8BQ_GLOBAL float*)amax)[i], s, r);
    ((FP8BQ_GLOBAL float*)scale)[i] = s;
  }
}

// ---------------------------------------------------------------- dequantization
//
// The consumer side of the descale: x_hat = decode(q) * s, rounded once to
// fp32, optionally rounded again to BF16 (nearest, ties to even).  HBM-bound:
// 1 byte read and 4 (fp32) or 2 (BF16) bytes written per element.

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum OutType : int { kOutF32 = 0, kOutBF16 = 1 };

// Round a finite fp32 value to BF16 bits, nearest with ties to even: adding
// 0x7FFF plus the kept LSB to the 16 dropped bits carries into the kept part
// exactly when they are above half, or exactly half with an odd kept LSB.
__device__ __forceinline__ uint32_t bf16_rne(float y) {
  const uint32_t b = __float_as_uint(y);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Four e4m3fn bytes of one dword -> four floats times s.
__device__ __forceinline__ f32x4 dq4(uint32_t w, float s) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4{lo.x * s, lo.y * s, hi.x * s, hi.y * s};
}

// Vector dequantization: every lane writes one 16-byte output chunk per
// group -- 4 codes to 4 fp32, or 8 codes to 8 BF16 -- so each wave store is
// one contiguous 1 KB run (16 B per lane, lanes adjacent).  A workgroup
// handles blocks of kDqUnroll * 256 consecutive groups, all loads issued
// before the stores.  Full blocks take a body without any branch: with a
// per-lane guard around each load, the compiler's wait counting at the joins
// made the second group's loads wait for the first group's data (measured:
// fp32 output 68% -> 76% of the HBM peak, BF16 76% -> 78%).
// Needs N % G == 0, bn % G == 0 (a group never straddles a row or a tile),
// q aligned to G bytes and out to 16 bytes (G = 4 for fp32, 8 for BF16).
//
// Index math: (row0, col0) of a block's first group is divided out once per
// workgroup and then advanced by the grid stride (step_rows, step_cols);
// inside a block every numerator is below 2^31, so group -> row, column and
// tile indices are multiply-and-shift divisions by the invariant gpr (groups
// per row), bm and bn.
constexpr int kDqUnroll = 2;

// One block of kThreads * kDqUnroll groups starting at group b0 = (row0,
// col0).  Every lane issues all its loads before any store; with TAIL (the
// block runs past the last group) lanes past the end read the last group
// (clamped indices) and store nothing.  Without TAIL the body has no branch,
// so no wait separates the loads.
template <int OUT, bool TAIL>
__device__ __forceinline__ void dequant_block(const uint8_t* __restrict__ q,
                                              const float* __restrict__ s, int32_t gpr, int32_t TN,
                                              Div31 by_gpr, Div31 by_bm, Div31 by_bn,
                                              void* __restrict__ out, int64_t groups,
                                              int32_t last_row, int64_t b0, int64_t row0,
                                              int32_t col0) {
  constexpr int G = OUT == kOutF32 ? 4 : 8;
  typedef typename std::conditional<G == 4, uint32_t, u32x2>::type QWord;
  QWord w[kDqUnroll];
  float sc[kDqUnroll];
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const uint32_t o = threadIdx.x + k * kThreads;
    const int64_t g = b0 + o;
    // col0 < gpr < 2^29 and o < 256 * kDqUnroll: c < 2^31; col * G < N.
    const uint32_t c = (uint32_t)col0 + o;
    const uint32_t dr = div31(c, by_gpr);
    const uint32_t col = c - dr * (uint32_t)gpr;
    uint32_t row = (uint32_t)row0 + dr;
    int64_t gl = g;
    if (TAIL) {
      row = min(row, (uint32_t)last_row);
      gl = g < groups ? g : groups - 1;
    }
    w[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL QWord*)(q) + gl);
    sc[k] = ((const FP8BQ_GLOBAL float*)s)[(int64_t)div31(row, by_bm) * TN + div31(col * G, by_bn)];
  }
#pragma unroll
  for (int k = 0; k < kDqUnroll; ++k) {
    const int64_t g = b0 + threadIdx.x + k * kThreads;
    if (TAIL && g >= groups) continue;
    if constexpr (OUT == kOutF32) {
      __builtin_nontemporal_store(dq4(w[k], sc[k]), (FP8BQ_GLOBAL f32x4*)out + g);
    } else {
      const f32x4 a = dq4(w[k].x, sc[k]);
      const f32x4 b = dq4(w[k].y, sc[k]);
      const u32x4 p{bf16_rne(a.x) | (bf16_rne(a.y) << 16), bf16_rne(a.z) | (bf16_rne(a.w) << 16),
                    bf16_rne(b.x) | (bf16_rne(b.y) << 16), bf16_rne(b.z) | (bf16_rne(b.w) << 16)};
      __builtin_nontemporal_store(p, (FP8BQ_GLOBAL u32x4*)out + g);
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_vec(const uint8_t* __restrict__ q,
                                                        const float* __restrict__ s, int32_t gpr,
                                                        int32_t TN, Div31 by_gpr, Div31 by_bm,
                                                        Div31 by_bn, void* __restrict__ out,
                                                        int64_t groups, int32_t last_row,
                                                        int64_t step_rows, int32_t step_cols) {
  const int64_t per_block = (int64_t)kThreads * kDqUnroll;
  int64_t b0 = (int64_t)blockIdx.x * per_block;
  if (b0 >= groups) return;
  int64_t row0 = b0 / gpr;            // once per workgroup
  int32_t col0 = (int32_t)(b0 - row0 * gpr);
  for (;;) {
    if (b0 + per_block <= groups) {
      dequant_block<OUT, false>(q, s, gpr, TN, by_gpr, by_bm, by_bn, out, groups, last_row, b0,
                                row0, col0);
    } else {
      dequant_block<OUT, true>(q, s, gpr, TN, by_gpr, by_bm, by_bn, out, groups, last_row, b0,
                               row0, col0);
    }
    b0 += (int64_t)gridDim.x * per_block;
    if (b0 >= groups) break;
    row0 += step_rows;
    col0 += step_cols;
    if (col0 >= gpr) {
      col0 -= gpr;
      ++row0;
    }
  }
}

// A list of tensors that take the vector body, in one launch: the table
// rides in the kernel arguments.  Unit u is one block of one tensor: the
// entry whose first unit start[e] is the largest <= u.  Dequantization
// units are small (a few KB each), so the search that finds the entry is a
// measurable share of a unit's life: it runs in two rounds of independent
// uniform loads -- 15 entries of a contiguous coarse table (start[16 k])
// pick a bucket of 16 entries, then those 15 entries pick the entry -- where
// a binary search makes eight dependent loads.  Entries past the table hold
// INT32_MAX, so neither round compares against the count.  The block's
// first group is divided into (row, column) once (32-bit: the host keeps
// every entry below 2^31 groups).  Lists of at most 16 entries use a table
// of one bucket (one round of loads), and a list of one tensor no search at
// all (151937x4096 alone, fp32 out: 75.5% with the two rounds).  Measured
// on MI355X, % of the HBM peak
// (dense 36-layer set / 8 MoE layers / the 151937x4096 matrix alone), one
// grouped call, fp32 out | BF16 out:
//   two-level search, 1 block per unit:       79.6 / 77.7 / 79.0 | 79.5 / 80.6 / 81.3  (taken)
//   binary search, 1 block per unit:          68.5 / 70.1 / 80.6 | 79.8 / 79.1 / 77.8
//   binary search, runs of 2 blocks per unit: 73.9 / 74.2 / 75.9 | 71.7 / 73.5 / 74.0
//   two-level, 4 or 8 groups per thread:      68.5, 66.2 on the dense set (fp32)
//   two-level, runs of 2 (2 / 4 groups):      73.7 / 70.2 on the dense set (fp32)
// Also slower: the first two-level form, whose rounds the compiler split
// into five dependent batches of loads (55% fp32 on the dense set), and
// counting the entries with one ballot per four table entries per lane
// (vector loads of the kernel-argument table: 55-61%).
struct DqEntry {
  const uint8_t* q;
  const float* s;
  void* out;
  int64_t groups;     // M * N / G, < 2^31
  int32_t gpr;        // groups per row, N / G
  int32_t TN;
  int32_t last_row;   // M - 1
  int32_t step_rows;  // one block of groups = step_rows rows + step_cols groups
  int32_t step_cols;
  Div31 by_gpr;
  Div31 by_bm;
  Div31 by_bn;
};

constexpr int kDqArgsMax = 256;
constexpr int kDqBucket = 16;   // table entries per bucket of the two-level search

template <int CAP>
struct DqGroupArgs {
  int32_t coarse[CAP / kDqBucket];  // start[16 k]; INT32_MAX past the table
  int32_t start[CAP + kDqBucket];   // first unit of each entry, start[count] = total, then INT32_MAX
  DqEntry e[CAP];
};

// Entry owning unit u (start[0] = 0 <= u < start[count]; start strictly
// increasing, INT32_MAX past start[count]; units < 2^31).  A table of one
// bucket (CAP 16) takes one round of loads.
template <int CAP>
__device__ __forceinline__ int find_entry_2level(const int32_t* coarse, const int32_t* start,
                                                 int32_t u) {
  static_assert(CAP % kDqBucket == 0 && CAP <= kDqBucket * kDqBucket, "at most 16 buckets");
  int j = 0;
#pragma unroll
  for (int k = 1; k < CAP / kDqBucket; ++k) j += (int)(coarse[k] <= u);
  const int b = kDqBucket * j;
  int i = b;
#pragma unroll
  for (int k = 1; k < kDqBucket; ++k) i += (int)(start[b + k] <= u);
  return i;
}

// Lists of up to 16 entries take CAP 16, longer ones CAP 256; a list of one
// tensor skips the search.
template <int OUT, int CAP>
__global__ __launch_bounds__(kThreads) void dequant_group(const DqGroupArgs<CAP> a, int32_t count,
                                                          int32_t total) {
  const int64_t per_block = (int64_t)kThreads * kDqUnroll;
  for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int i = count == 1 ? 0 : find_entry_2level<CAP>(a.coarse, a.start, (int32_t)u);
    const DqEntry& e = a.e[i];
    const int64_t b0 = (u - a.start[i]) * per_block;
    const int64_t row0 = div31((uint32_t)b0, e.by_gpr);
    const int32_t col0 = (int32_t)(b0 - row0 * e.gpr);
    if (b0 + per_block <= e.groups) {
      dequant_block<OUT, false>(e.q, e.s, e.gpr, e.TN, e.by_gpr, e.by_bm, e.by_bn, e.out,
                                e.groups, e.last_row, b0, row0, col0);
    } else {
      dequant_block<OUT, true>(e.q, e.s, e.gpr, e.TN, e.by_gpr, e.by_bm, e.by_bn, e.out,
                               e.groups, e.last_row, b0, row0, col0);
    }
  }
}

// One thread per element: any shape, block size and alignment.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dequant_elem(const uint8_t* __restrict__ q,
                                                         const float* __restrict__ s, int64_t N,
                                                         int32_t bm, int32_t bn, int32_t TN,
                                                         void* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += stride) {
    const int64_t row = e / N;
    const int64_t col = e - row * N;
    const float sc = ((const FP8BQ_GLOBAL float*)s)[(row / bm) * TN + col / bn];
    const f32x2 v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)((const FP8BQ_GLOBAL uint8_t*)q)[e], false);
    const float v = v2[0];
    const float y = v * sc;
    if constexpr (OUT == kOutF32) {
      ((FP8BQ_GLOBAL float*)out)[e] = y;
    } else {
      ((FP8BQ_GLOBAL uint16_t*)out)[e] = (uint16_t)bf16_rne(y);
    }
  }
}

// ---------------------------------------------------------------- grouped launch, table in the arguments
//
// Groups of up to kArgsMax tensors pass their descriptor table by value in
// the kernel arguments, so the launch needs no host-to-device copy (and no
// workspace).  The table is read with uniform scalar loads like any other
// kernel argument.

constexpr int kArgsMax = 512;

struct ArgTensor {
  const uint16_t* x;
  uint8_t* q;
  float* s;
  int32_t M;
  int32_t N;
  int32_t body;     // Body of this tensor
  int32_t pad;
};

template <int CAP>
struct GroupArgs {
  int32_t start[CAP + 1];  // first unit of each tensor; start[count] = total
  ArgTensor t[CAP];
};

template <int KIND, int CAP>
__global__ __launch_bounds__(kThreads) void quantize_group_args(const GroupArgs<CAP> a,
                                                                int32_t count, int32_t bm,
                                                                int32_t bn, int32_t total) {
  __shared__ uint32_t red[32];
  for_each_unit(total, [&](int64_t u) {
    const int lo = find_tensor(a.start, count, u);
    const ArgTensor& at = a.t[lo];
    Desc d;
    d.x = at.x;
    d.q = at.q;
    d.s = at.s;
    d.M = at.M;
    d.N = at.N;
    d.TN = (int32_t)(((int64_t)at.N + bn - 1) / bn);
    d.body = at.body;
    constexpr int64_t kUnitCols = KIND == kT128W || KIND == kT64W ? 512 : 128;
    d.UN = at.body != kBodyVec ? d.TN : (int32_t)(((int64_t)at.N + kUnitCols - 1) / kUnitCols);
    d.pad = 0;
    d.reserved = 0;
    run_unit<KIND>(d, bm, bn, u - a.start[lo], red);
  });
}

// ---------------------------------------------------------------- grouped shards, table in the arguments
//
// A list of shards that share one block size and take the small-tile
// kernels, in one launch per pass: unit u belongs to the entry whose first
// unit start[e] is the largest <= u (units: local tiles, or 64-row units
// for one-row tiles).

constexpr int kShardArgsMax = 512;

struct ShardEntry {
  const uint16_t* x;
  uint8_t* q;
  const float* amax;  // pass 1: the given maxima
  float* out;         // pass 0: the maxima; pass 1: the scales (may be amax)
  int32_t M;
  int32_t N;
  int32_t row_phase;
  int32_t col_phase;
};

template <int CAP>
struct ShardGroupArgs {
  int32_t start[CAP + 1];
  ShardEntry e[CAP];
};

template <int PASS, bool ROWS, int CAP>
__global__ __launch_bounds__(kThreads) void shard_group(const ShardGroupArgs<CAP> a, int32_t count,
                                                        int32_t bm, int32_t bn, int32_t total) {
  __shared__ uint32_t red[32];
  for_each_unit(total, [&](int64_t u) {
    const int i = find_tensor(a.start, count, u);
    const ShardEntry& en = a.e[i];
    Big b;
    b.x = en.x;
    b.q = en.q;
    b.M = en.M;
    b.N = en.N;
    b.bm = bm;
    b.bn = bn;
    b.row_phase = en.row_phase;
    b.col_phase = en.col_phase;
    b.TMl = ((int64_t)en.row_phase + en.M + bm - 1) / bm;
    b.TNl = ((int64_t)en.col_phase + en.N + bn - 1) / bn;
    b.cpt = 1;
    b.items = b.TMl * b.TNl;
    b.flat = 0;
    b.vec = 1;
    b.cpm = 1;
    b.pad = 0;
    const int64_t lu = u - a.start[i];
    if constexpr (ROWS) {
      shard_rows_unit<PASS>(b, lu, en.amax, en.out);
    } else {
      shard_small_tile<PASS>(b, lu, en.amax, en.out, red);
    }
  });
}

// [128,128] shards, quantize pass, four side-by-side whole tiles per unit
// (128 x 512, the layout of the four-tile quantize unit): thread t of wave w
// holds columns 8(t%64)..+7 of rows w, w+4, ..., w+124; the four given
// maxima are read into LDS before the barrier, so `amax` may be `out`.
__device__ __forceinline__ void shard_wide_quant(const Big& b, int64_t ti, int64_t g,
                                                 const float* amax, float* out, uint32_t* red) {
  constexpr int L = 32;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int sub = lane >> 4;
  const int64_t N = b.N;
  const int64_t r0 = ti * 128 - b.row_phase;
  const int64_t c0 = g * 512 - b.col_phase;
  const int64_t tile0 = ti * b.TNl + g * 4;
  if (t < 4) red[8 + t] = __float_as_uint(((const FP8BQ_GLOBAL float*)amax)[tile0 + t]);
  const size_t base = (size_t)(r0 + wave) * (size_t)N + (size_t)(c0 + lane * 8);
  const FP8BQ_GLOBAL u32x4* xp = (const FP8BQ_GLOBAL u32x4*)(b.x + base);
  const size_t pitch16 = (size_t)N * 4 / 8;
  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) v[k] = __builtin_nontemporal_load(&xp[k * pitch16]);
  __syncthreads();
  float s, r;
  tile_scale_f(__uint_as_float(red[8 + sub]), s, r);
  FP8BQ_GLOBAL u32x2* qp = (FP8BQ_GLOBAL u32x2*)(b.q + base);
  const size_t qpitch8 = (size_t)N * 4 / 8;
#pragma unroll
  for (int k = 0; k < L; ++k) __builtin_nontemporal_store(quant8(v[k], r), &qp[k * qpitch8]);
  if (wave == 0 && (lane & 15) == 0) ((FP8BQ_GLOBAL float*)out)[tile0 + sub] = s;
}

// The same unit when some of its 128 rows lie outside the shard (the first
// or last local tile row of a shard at a row phase, or of a shard shorter
// than a tile row) but its 512 columns lie inside: rows outside [0, M) are
// neither read nor written, and the four given maxima scale the others.
// Edge slabs of row shards (64 of 128 rows at phase 64) went from one tile
// at a time to this body.
__device__ __forceinline__ void shard_wide_quant_rows(const Big& b, int64_t ti, int64_t g,
                                                      const float* amax, float* out,
                                                      uint32_t* red) {
  constexpr int L = 32;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int sub = lane >> 4;
  const int64_t N = b.N;
  const int64_t r0 = ti * 128 - b.row_phase;
  const int64_t col = g * 512 - b.col_phase + lane * 8;
  const int64_t tile0 = ti * b.TNl + g * 4;
  if (t < 4) red[8 + t] = __float_as_uint(((const FP8BQ_GLOBAL float*)amax)[tile0 + t]);
  u32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const int64_t row = r0 + wave + 4 * k;
    v[k] = u32x4{0u, 0u, 0u, 0u};
    if (row >= 0 && row < b.M) {
      v[k] = __builtin_nontemporal_load((const FP8BQ_GLOBAL u32x4*)(b.x + row * N + col));
    }
  }
  __syncthreads();
  float s, r;
  tile_scale_f(__uint_as_float(red[8 + sub]), s, r);
#pragma unroll
  for (int k = 0; k < L; ++k) {
    const int64_t row = r0 + wave + 4 * k;
    if (row >= 0 && row < b.M) {
      __builtin_nontemporal_store(quant8(v[k], r), (FP8BQ_GLOBAL u32x2*)(b.q + row * N + col));
    }
  }
  if (wave == 0 && (lane & 15) == 0) ((FP8BQ_GLOBAL float*)out)[tile0 + sub] = s;
}

// Quantize pass of grouped [128,128] shards in four-tile units: unit (ti, g)
// covers local tiles (ti, 4g..4g+3); units whose four tiles lie whole inside
// the shard take shard_wide_quant, units whose columns do take
// shard_wide_quant_rows, the others their tiles one by one.  The maxima pass
// keeps one tile per unit even for shards one tile row deep: the same
// four-tile units with rows masked measured slower there (MoE row shards
// 68.3% -> 67.7%, dense set unchanged).  At 2
// workgroups per CU, against one tile per workgroup at 4: the 151937x4096
// shard at phase (64, 0) 77.0% -> 78.5% of peak, at (0, 64) 65.5% -> 72.9%,
// 70 dense-set shards at (64, 0) 76.9% -> 79.0% (3 per CU: 77.2 / 70.5 / 77.9%).
template <int CAP>
__global__ __launch_bounds__(kThreads) void shard_group_wide(const ShardGroupArgs<CAP> a,
                                                             int32_t count, int32_t total) {
  __shared__ uint32_t red[32];
  for_each_unit(total, [&](int64_t u) {
    const int i = find_tensor(a.start, count, u);
    const ShardEntry& en = a.e[i];
    Big b;
    b.x = en.x;
    b.q = en.q;
    b.M = en.M;
    b.N = en.N;
    b.bm = 128;
    b.bn = 128;
    b.row_phase = en.row_phase;
    b.col_phase = en.col_phase;
    b.TMl = ((int64_t)en.row_phase + en.M + 127) / 128;
    b.TNl = ((int64_t)en.col_phase + en.N + 127) / 128;
    b.cpt = 1;
    b.items = b.TMl * b.TNl;
    b.flat = 0;
    b.vec = 1;
    b.cpm = 1;
    b.pad = 0;
    const int64_t lu = u - a.start[i];
    const int64_t groups = (b.TNl + 3) / 4;
    const int64_t ti = lu / groups;
    const int64_t g = lu - ti * groups;
    const int64_t r0 = ti * 128 - b.row_phase;
    const int64_t c0 = g * 512 - b.col_phase;
    if (r0 >= 0 && r0 + 128 <= b.M && c0 >= 0 && c0 + 512 <= b.N) {
      shard_wide_quant(b, ti, g, en.amax, en.out, red);
    } else if (c0 >= 0 && c0 + 512 <= b.N) {
      shard_wide_quant_rows(b, ti, g, en.amax, en.out, red);
    } else {
      for (int64_t tj = g * 4; tj < g * 4 + 4 && tj < b.TNl; ++tj) {
        if (tj > g * 4) __syncthreads();  // red[] of the previous tile is read
        shard_small_tile<1>(b, ti * b.TNl + tj, en.amax, en.out, red);
      }
    }
  });
}

// A list of [1,128] tensors that all have flat units (see quantize_flat_one).
template <int CAP>
__global__ __launch_bounds__(kThreads) void quantize_group_args_flat(const GroupArgs<CAP> a,
                                                                     int32_t count,
                                                                     int32_t total) {
  for_each_unit(total, [&](int64_t u) {
    const int lo = find_tensor(a.start, count, u);
    const ArgTensor& at = a.t[lo];
    Desc d;
    d.x = at.x;
    d.q = at.q;
    d.s = at.s;
    d.M = at.M;
    d.N = at.N;
    d.TN = at.N / 128;
    d.UN = d.TN;
    d.body = kBodyFlat;
    d.pad = 0;
    d.reserved = 0;
    flat_r128(d, u - a.start[lo]);
  });
}

// The final cast alone: clamp and convert n floats.
__global__ __launch_bounds__(kThreads) void encode_e4m3(const float* __restrict__ y,
                                                        uint8_t* __restrict__ q, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    q[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(y[i]), 0.0f, 0, false) & 0xFF);
  }
}

}  // namespace fp8bq
