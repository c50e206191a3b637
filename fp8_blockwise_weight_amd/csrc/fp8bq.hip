// Host side of fp8bq: the C ABI declared in include/fp8bq.h.
//
// Every argument check runs before the first HIP call, so invalid calls are
// rejected without touching a device.  Compute calls enqueue on the caller's
// stream and return without synchronizing; nothing here allocates device
// memory.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "fp8bq.h"
#include "kernels.hpp"

// Device memory of fp8bq_quantize_many_noalloc: the descriptor table of a
// grouped call of more than FP8BQ_MANY_ARGS_MAX tensors (64-byte entries,
// then the int64 unit prefix sums), laid out as in a caller's workspace.
// Each device holds its own copy for the life of the process.  Host code
// never passes this name to a kernel (on the host it is a stand-in, not a
// device address): it uses the address hipGetSymbolAddress gives per device.
constexpr size_t kScratchBytes =
    (sizeof(fp8bq::Desc) * FP8BQ_NOALLOC_MAX_TENSORS + 255) / 256 * 256 +
    (sizeof(int64_t) * (FP8BQ_NOALLOC_MAX_TENSORS + 1) + 255) / 256 * 256;
static_assert(sizeof(fp8bq::Desc) == 64 && kScratchBytes == 1179904,
              "include/fp8bq.h states the size of this block");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using fp8bq::Desc;

thread_local int g_last_hip_error = 0;

int hip_failed(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return FP8BQ_ERR_HIP;
}

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxUnits = INT32_MAX;  // work units per tensor (32-bit unit math)
// Workgroups per launch: a dispatch counts at most 2^32 - 1 work-items.
// Kernels whose work exceeds the grid cover it in grid-sized rounds.
constexpr int64_t kMaxGrid = static_cast<int64_t>(UINT32_MAX) / fp8bq::kThreads;

// Dynamic LDS reserved (and left unused) by the vectorized quantize launches
// to cap how many workgroups share a CU (160 KB of LDS per gfx950 CU), i.e.
// how many bytes are in flight per CU.  Measured on MI355X:
//   [128,128], 32 KB per unit: 4 per CU is best (dense 36-layer set 76.0% ->
//     77.1% of peak; per-layer MoE launches 73.6% -> 76.5%);
//   [64,64] and [1,128], 16 KB per unit: 6 per CU is best (151937x4096:
//     [64,64] 75% at 4 per CU -> 79.6%, [1,128] 74% -> 77.5%).
constexpr unsigned kLds4PerCu = 36 * 1024;  // 160 KB / 36 KB -> 4 workgroups
constexpr unsigned kLds6PerCu = 26 * 1024;  // 160 KB / 26 KB -> 6 workgroups
constexpr unsigned kLds3PerCu = 44 * 1024;  // 160 KB / 44 KB -> 3 workgroups
constexpr unsigned kLds2PerCu = 64 * 1024;  // 160 KB / 64 KB -> 2 workgroups

// The wide [128,128] unit needs no reserve: its ~224 VGPRs already hold a
// CU to 2 workgroups (128 KB of tile data each in flight); a 96 KB reserve
// (1 per CU) took the dense 36-layer set from 80.9% to 72.9%.  The wide [64,64]
// unit (64 KB per workgroup, ~95 VGPRs) runs best at 2 per CU in launches of
// up to 8 tensors (151937x4096: 82.4%, against 80.9% at 3 and 79.6% at 4)
// and at 3 per CU with larger tables (dense 36-layer set: 81.0%, 75.8% at
// 2), whose per-unit table search needs the extra waves.
constexpr unsigned lds_for(int kind, int32_t count = 1) {
  return kind == fp8bq::kT64W ? (count <= 8 ? kLds2PerCu : kLds3PerCu)
         : kind == fp8bq::kGeneral || kind == fp8bq::kT128W
             ? 0u
             : (kind == fp8bq::kT128 ? kLds4PerCu : kLds6PerCu);
}

// [128,128] launches take the wide unit (kT128W, four tiles per workgroup),
// and [64,64] launches theirs (kT64W, eight tiles), when every vector-body
// tensor is a whole number of 512-column units wide
// (no half-empty units) and the launch has at least kWideMinUnits of them
// (16 rounds of the 512 workgroups the chip holds), so that the 4x larger
// units still spread evenly.  Measured: the dense 36-layer set 77.1% ->
// 80.3%, the 151937x4096 matrix 75.7% -> 77.4%; a 12288x4096 tensor alone
// (768 wide units), an MoE layer with its 768-wide matrices and the
// 4097x11008 matrix are faster with the one-tile unit.
constexpr int64_t kWideMinUnits = 8192;

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_state[kMaxDevices];

int device_check() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failed(e);
  int state = (dev >= 0 && dev < kMaxDevices) ? g_arch_state[dev].load(std::memory_order_acquire) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_failed(e);
    const char* arch = prop.gcnArchName;
    const bool ok = std::strncmp(arch, "gfx950", 6) == 0 && (arch[6] == '\0' || arch[6] == ':');
    state = ok ? 1 : 2;
    if (dev >= 0 && dev < kMaxDevices) g_arch_state[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8BQ_OK : FP8BQ_ERR_UNSUPPORTED_DEVICE;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

int kind_of(int32_t bm, int32_t bn) {
  if (bm == 128 && bn == 128) return fp8bq::kT128;
  if (bm == 64 && bn == 64) return fp8bq::kT64;
  if (bm == 1 && bn == 128) return fp8bq::kR128;
  return fp8bq::kGeneral;
}

// Wide units (128 or 64 rows x 512 columns) of one tensor: 0 when it takes a
// general body (it does not constrain the choice), -1 when its width is not
// a whole number of 512-column units.
int64_t wide_units(const void* x, int64_t M, int64_t N, const void* q, int64_t rows = 128) {
  if (M <= 0 || N <= 0) return 0;
  const bool aligned = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(q) & 7) == 0;
  if (!aligned) return 0;
  if (N % 512 != 0) return -1;
  return ceil_div(M, rows) * (N / 512);
}

// The wide kind of a [128,128] or [64,64] launch whose tensors' wide-unit
// counts (wide_units) sum to `wide` (negative: some width is not a whole
// number of 512-column units), or `kind` itself.
int wide_kind(int kind, int64_t wide) {
  if (wide < kWideMinUnits) return kind;
  return kind == fp8bq::kT128 ? fp8bq::kT128W : (kind == fp8bq::kT64 ? fp8bq::kT64W : kind);
}

// Checks one tensor and fills its descriptor.  Returns FP8BQ_OK with
// *units = 0 for an empty tensor.
int make_desc(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, void* q, float* s,
              int kind, Desc* d, int64_t* units) {
  *units = 0;
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (M == 0 || N == 0) return FP8BQ_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const uintptr_t qa = reinterpret_cast<uintptr_t>(q);
  const uintptr_t sa = reinterpret_cast<uintptr_t>(s);
  if ((xa & 1) != 0 || (sa & 3) != 0) return FP8BQ_ERR_INVALID_ARGUMENT;
  const int64_t TM = ceil_div(M, bm);
  const int64_t TN = ceil_div(N, bn);
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(N);
  const uint64_t ns = static_cast<uint64_t>(TM) * static_cast<uint64_t>(TN);
  if (overlap(x, 2 * n, q, n) || overlap(x, 2 * n, s, 4 * ns) || overlap(q, n, s, 4 * ns)) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  const bool aligned = (N % 8) == 0 && (xa & 15) == 0 && (qa & 7) == 0;
  const bool vec = kind != fp8bq::kGeneral && aligned;
  // 8-aligned tile columns: a whole tile in registers up to kRegTile elements,
  // two vector passes above that.
  const bool colvec = aligned && (bn % 8) == 0;
  const bool reg = colvec && static_cast<int64_t>(bm) * static_cast<int64_t>(bn) <= fp8bq::kRegTile;
  d->x = static_cast<const uint16_t*>(x);
  d->q = static_cast<uint8_t*>(q);
  d->s = s;
  d->M = M;
  d->N = N;
  d->TN = static_cast<int32_t>(TN);
  d->pad = 0;
  d->reserved = 0;
  int64_t u;
  if (vec && kind == fp8bq::kR128 && (N % 128) == 0) {
    // [1,128] tiles are consecutive 128-element runs: 64 of them per unit
    d->UN = static_cast<int32_t>(TN);
    d->body = fp8bq::kBodyFlat;
    u = ceil_div(M * (N / 128), 64);
  } else if (vec) {
    const int64_t rows = kind == fp8bq::kT128 || kind == fp8bq::kT128W ? 128 : 64;
    d->UN = static_cast<int32_t>(ceil_div(N, kind == fp8bq::kT128W || kind == fp8bq::kT64W ? 512 : 128));
    d->body = fp8bq::kBodyVec;
    u = ceil_div(M, rows) * d->UN;
  } else {
    if (TN > INT32_MAX) return FP8BQ_ERR_INVALID_ARGUMENT;
    d->UN = static_cast<int32_t>(TN);
    d->body = reg ? fp8bq::kBodyRegTile : (colvec ? fp8bq::kBodyLoopVec : fp8bq::kBodyScalar);
    if (TM > kMaxUnits / TN) return FP8BQ_ERR_INVALID_ARGUMENT;
    u = TM * TN;
  }
  if (u > kMaxUnits) return FP8BQ_ERR_INVALID_ARGUMENT;
  *units = u;
  return FP8BQ_OK;
}

unsigned grid_for(int64_t units) {
  return static_cast<unsigned>(units < kMaxGrid ? units : kMaxGrid);
}

// Flat [1,128] units stream 16 KB contiguous runs; they run best at 4
// workgroups per CU (151937x4096: 80.6% at 6 per CU, 83.1% at 4), while the
// 64-row [1,128] units of other widths keep 6 per CU.
bool is_flat(const Desc& d) { return d.body == fp8bq::kBodyFlat; }

// LDS reserve of a launch whose tensors all have flat bodies (all_flat) or not.
unsigned lds_of(int kind, bool all_flat, int32_t count = 1) {
  return kind == fp8bq::kR128 && all_flat ? kLds4PerCu : lds_for(kind, count);
}

bool all_flat(const std::vector<Desc>& ds) {
  for (const Desc& d : ds) {
    if (!is_flat(d)) return false;
  }
  return !ds.empty();
}

template <int KIND>
void launch_one(const Desc& d, int32_t bm, int32_t bn, int64_t units, hipStream_t st) {
  if (is_flat(d)) {
    hipLaunchKernelGGL(fp8bq::quantize_flat_one, dim3(grid_for(units)), dim3(fp8bq::kThreads),
                       kLds4PerCu, st, d, units);
    return;
  }
  hipLaunchKernelGGL(fp8bq::quantize_one<KIND>, dim3(grid_for(units)), dim3(fp8bq::kThreads),
                     lds_of(KIND, is_flat(d)),
                     st, d, bm, bn, units);
}

template <int KIND>
void launch_group(const Desc* descs, const int64_t* start, int32_t count, int32_t bm, int32_t bn,
                  int64_t units, unsigned lds, hipStream_t st) {
  hipLaunchKernelGGL(fp8bq::quantize_group<KIND>, dim3(grid_for(units)), dim3(fp8bq::kThreads),
                     lds, st, descs, start, count, bm, bn, units);
}

// Effective tile of an [M, N] tensor: more than kBigTile elements takes the
// two-pass path.
bool big_tiles(int64_t M, int64_t N, int32_t bm, int32_t bn) {
  const int64_t rows = M < bm ? M : bm;
  const int64_t cols = N < bn ? N : bn;
  return rows * cols > fp8bq::kBigTile;
}

// Chunks per pass-1 item for about `target` items, between 1 and
// kChunksPerMax.  Pass 2 does not depend on it.
fp8bq::Big with_cpm(fp8bq::Big b, int64_t target) {
  const int64_t per = b.items / target;
  b.cpm = static_cast<int32_t>(per < 1 ? 1 : (per > fp8bq::kChunksPerMax ? fp8bq::kChunksPerMax : per));
  return b;
}

// Describes a sub-matrix at tile phase (rp, cp) for the two-pass kernels.
fp8bq::Big make_big(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, int32_t rp,
                    int32_t cp, void* q) {
  fp8bq::Big b;
  b.x = static_cast<const uint16_t*>(x);
  b.q = static_cast<uint8_t*>(q);
  b.M = M;
  b.N = N;
  b.bm = bm;
  b.bn = bn;
  b.row_phase = rp;
  b.col_phase = cp;
  b.TMl = ceil_div(rp + M, bm);
  b.TNl = ceil_div(cp + N, bn);
  b.flat = (cp == 0 && bn >= N) ? 1 : 0;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const uintptr_t qa = reinterpret_cast<uintptr_t>(q);
  b.vec = ((N % 8) == 0 && (xa & 15) == 0 && (qa & 7) == 0) ? 1 : 0;
  const int64_t rows_max = M < bm ? M : bm;
  const int64_t cols_max = N < bn ? N : bn;
  if (b.flat) {
    b.cpt = ceil_div(rows_max * N, fp8bq::kChunk);
  } else {
    const int64_t rows_per = cols_max >= fp8bq::kChunk ? 1 : fp8bq::kChunk / cols_max;
    b.cpt = ceil_div(rows_max, rows_per);
  }
  b.items = b.TMl * b.TNl * b.cpt;
  b.cpm = 1;
  b.pad = 0;
  return with_cpm(b, fp8bq::kMaxItemsTarget);
}

// Pass-1 items of a large-tile sub-matrix.
int64_t big_max_items(const fp8bq::Big& b) { return b.TMl * b.TNl * ceil_div(b.cpt, b.cpm); }

unsigned grid_capped(int64_t n, int64_t per_block) {
  const int64_t blocks = (n + per_block - 1) / per_block;
  return static_cast<unsigned>(blocks < 65536 * 16 ? (blocks < 1 ? 1 : blocks) : 65536 * 16);
}

// Shards: pass 1 with atomic maxima into `amax` (zeroed first), with fewer,
// larger items than the slot form: 4096x4096 as one tile took 28 us at
// ~2048 items and 17 us at ~256 on MI355X.
void launch_big_amax(const fp8bq::Big& b, float* amax, hipStream_t st) {
  const fp8bq::Big a = with_cpm(b, fp8bq::kAtomicItemsTarget);
  const int64_t nt = a.TMl * a.TNl;
  hipLaunchKernelGGL(fp8bq::fill_zero, dim3(grid_capped(nt, fp8bq::kThreads)), dim3(fp8bq::kThreads),
                     0, st, reinterpret_cast<uint32_t*>(amax), nt);
  const int64_t items = big_max_items(a);
  hipLaunchKernelGGL(fp8bq::big_max<false>, dim3(grid_for(items)), dim3(fp8bq::kThreads), 0, st, a,
                     reinterpret_cast<uint32_t*>(amax), items);
}

// Shards: pass 2 with given maxima, then the scales.  `amax` may be
// `scale_inv` itself (converted in place after pass 2 has read it).
void launch_big_quant(const fp8bq::Big& b, const float* amax, float* scale_inv, hipStream_t st) {
  const int64_t nt = b.TMl * b.TNl;
  hipLaunchKernelGGL(fp8bq::big_quant<false>, dim3(grid_for(b.items)), dim3(fp8bq::kThreads), 0, st,
                     b, amax);
  hipLaunchKernelGGL(fp8bq::finalize_scales, dim3(grid_capped(nt, fp8bq::kThreads)),
                     dim3(fp8bq::kThreads), 0, st, amax, scale_inv, nt);
}

// Shards whose tiles hold at most kRegTile elements and whose tile columns
// start on 8-element boundaries take the one-workgroup-per-tile kernels
// (maxima stored directly, quantize and scales in one launch).
bool shard_small_ok(const fp8bq::Big& b) {
  const int64_t rows = b.M < b.bm ? b.M : b.bm;
  const int64_t cols = b.N < b.bn ? b.N : b.bn;
  return b.vec != 0 && (b.bn % 8) == 0 && (b.col_phase % 8) == 0 && rows * cols <= fp8bq::kRegTile;
}

// One-row tiles of at most 128 columns take 64-row units (16 row-tiles per
// wave) instead of one workgroup per tile.
bool shard_rows_ok(const fp8bq::Big& b) { return shard_small_ok(b) && b.bm == 1 && b.bn <= 128; }

// Pass 0: amax of every local tile into `out`.  Pass 1: quantize with the
// given `amax` and write the scales to `out` (which may be `amax`).
void launch_shard_small(int pass, const fp8bq::Big& b, const float* amax, float* out,
                        hipStream_t st) {
  if (shard_rows_ok(b)) {
    const int64_t units = ceil_div(b.M, 64) * b.TNl;
    if (pass == 0) {
      hipLaunchKernelGGL(fp8bq::shard_rows<0>, dim3(grid_for(units)), dim3(fp8bq::kThreads), 0, st,
                         b, amax, out, units);
    } else {
      hipLaunchKernelGGL(fp8bq::shard_rows<1>, dim3(grid_for(units)), dim3(fp8bq::kThreads), 0, st,
                         b, amax, out, units);
    }
    return;
  }
  const int64_t tiles = b.TMl * b.TNl;
  if (pass == 0) {
    hipLaunchKernelGGL(fp8bq::shard_small<0>, dim3(grid_for(tiles)), dim3(fp8bq::kThreads), 0, st,
                       b, amax, out, tiles);
  } else {
    // Full 16,384-element tiles quantize best at 4 workgroups per CU, as the
    // [128,128] unit does (151937x4096 shard: 72-74% -> 75.5% of peak);
    // smaller tiles run uncapped (8 KB tiles lose 20 points under that cap).
    const int64_t rows = b.M < b.bm ? b.M : b.bm;
    const int64_t cols = b.N < b.bn ? b.N : b.bn;
    const unsigned lds = rows * cols >= fp8bq::kRegTile ? kLds4PerCu : 0u;
    hipLaunchKernelGGL(fp8bq::shard_small<1>, dim3(grid_for(tiles)), dim3(fp8bq::kThreads), lds, st,
                       b, amax, out, tiles);
  }
}

// A whole tensor's pass-1 slots fit in its q buffer (from the first
// 4-byte-aligned byte).  Always true for tiles of more than kBigTile
// elements, since a slot covers at least one chunk; checked anyway.
bool big_slots_fit(const fp8bq::Big& b) {
  const uint64_t pad = (4 - (reinterpret_cast<uintptr_t>(b.q) & 3)) & 3;
  const uint64_t need = 4 * static_cast<uint64_t>(big_max_items(b)) + pad;
  return need <= static_cast<uint64_t>(b.M) * static_cast<uint64_t>(b.N);
}

// A whole tensor with large tiles: slots in q, tile scales, then pass 2.
void launch_big_tensor(const fp8bq::Big& b, float* scale_inv, hipStream_t st) {
  if (!big_slots_fit(b)) {
    // scale_inv doubles as the scratch for the per-tile maxima.
    launch_big_amax(b, scale_inv, st);
    launch_big_quant(b, scale_inv, scale_inv, st);
    return;
  }
  uint32_t* slots = fp8bq::big_slots(b.q);
  const int64_t items = big_max_items(b);
  const int64_t nt = b.TMl * b.TNl;
  hipLaunchKernelGGL(fp8bq::big_max<true>, dim3(grid_for(items)), dim3(fp8bq::kThreads), 0, st, b,
                     slots, items);
  hipLaunchKernelGGL(fp8bq::big_reduce, dim3(grid_for(nt)), dim3(fp8bq::kThreads), 0, st,
                     static_cast<const uint32_t*>(slots), ceil_div(b.cpt, b.cpm), scale_inv, nt);
  hipLaunchKernelGGL(fp8bq::big_quant<true>, dim3(grid_for(b.items)), dim3(fp8bq::kThreads), 0, st,
                     b, static_cast<const float*>(scale_inv));
}

// ---- one scale per tensor, held in registers (resident_quant)
//
// A whole tensor of at least kResMinValues values with one tile, aligned for
// 16-byte loads, that fits in the registers of the grid the device holds at
// once.  Grid and chunks per thread (L) per tensor, from measurements on
// MI355X: the fewest chunks per thread that need at most 128 workgroups
// (1024x4096: 128 x 16 chunks 8.6 us, 256 x 8 9.4 us, 512 x 4 12.5 us),
// else 32 or 48 chunks per thread (4096x4096: 256 x 32 14.5 us against
// 512 x 16 17.1 us; 12288x4096: 512 x 48 29.4 us).  The two-pass path took
// 10.6, 19.2 and 44.7 us.
constexpr int64_t kResMinValues = int64_t{1} << 20;
constexpr int kResGroupCap = 256;  // tensors per persistent resident launch
constexpr int kResPrepCap = kResGroupCap;
constexpr int64_t kResWaitUsDefault = 2000;

struct ResPlan {
  int L;
  uint32_t grid;
  uint32_t nchunks;
};

// Per device: workgroups of the resident kernels held at once (0 unknown,
// -1 failed) and s_memrealtime ticks per microsecond.
std::atomic<int> g_res_grid[kMaxDevices];
std::atomic<int> g_res_tick_mhz[kMaxDevices];
std::atomic<int64_t> g_res_wait_us{kResWaitUsDefault};

// Workgroups of the resident kernels the current device holds at once, or 0.
int resident_capacity(int* tick_mhz) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cap = g_res_grid[dev].load(std::memory_order_acquire);
  if (cap == 0) {
    int per = 0, per_group = 0, cus = 0, khz = 0;
    const bool ok =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fp8bq::resident_quant<fp8bq::kResMaxLoads>,
                                                     fp8bq::kThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_group, fp8bq::resident_group<kResGroupCap>,
                                                     fp8bq::kThreads, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess &&
        per > 0 && per_group > 0 && cus > 0 && khz >= 1000;
    (void)hipGetLastError();
    cap = ok ? (per < per_group ? per : per_group) * cus : -1;
    g_res_tick_mhz[dev].store(ok ? khz / 1000 : 0, std::memory_order_relaxed);
    g_res_grid[dev].store(cap, std::memory_order_release);
  }
  *tick_mhz = g_res_tick_mhz[dev].load(std::memory_order_relaxed);
  return cap > 0 ? cap : 0;
}

// The resident plan of a tensor (bm >= M and bn >= N: one tile), or false.
bool resident_plan(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, const void* q,
                   int cap, ResPlan* p) {
  if (cap <= 0 || M > bm || N > bn || (N % 8) != 0) return false;
  if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(q) & 7) != 0) {
    return false;
  }
  const int64_t n = M * N;
  if (n < kResMinValues) return false;
  const int64_t chunks = n / 8;
  if (chunks > (int64_t{1} << 26)) return false;  // byte offsets stay below 2^31
  const int64_t per_wg = fp8bq::kThreads;
  for (int L : {4, 8, 16}) {
    const int64_t g = ceil_div(chunks, per_wg * L);
    if (g <= 128 && g <= cap) {
      *p = ResPlan{L, static_cast<uint32_t>(g), static_cast<uint32_t>(chunks)};
      return true;
    }
  }
  for (int L : {32, fp8bq::kResMaxLoads}) {
    const int64_t g = ceil_div(chunks, per_wg * L);
    if (g <= cap) {
      *p = ResPlan{L, static_cast<uint32_t>(g), static_cast<uint32_t>(chunks)};
      return true;
    }
  }
  return false;
}

// Handshake words and scale sentinels of n resident tensors (before any of
// their resident_quant launches).
void launch_resident_prep(const fp8bq::ResTensor* ts, int n, hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kResPrepCap) {
    const int c = n - i0 < kResPrepCap ? n - i0 : kResPrepCap;
    fp8bq::ResPrepArgs<kResPrepCap> a;
    std::memset(&a, 0, sizeof(a));
    for (int i = 0; i < c; ++i) a.t[i] = ts[i0 + i];
    hipLaunchKernelGGL(fp8bq::resident_prep<kResPrepCap>, dim3(1), dim3(kResPrepCap), 0, st, a, c);
  }
}

uint64_t resident_wait_ticks(int tick_mhz) {
  return static_cast<uint64_t>(g_res_wait_us.load(std::memory_order_relaxed)) *
         static_cast<uint64_t>(tick_mhz);
}

void launch_resident(const ResPlan& p, const void* x, void* q, float* s, int tick_mhz,
                     hipStream_t st) {
  const uint64_t ticks = resident_wait_ticks(tick_mhz);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint8_t* qs = static_cast<uint8_t*>(q);
  const dim3 g(p.grid), b(fp8bq::kThreads);
  switch (p.L) {
    case 4: hipLaunchKernelGGL(fp8bq::resident_quant<4>, g, b, 0, st, xs, qs, s, p.nchunks, ticks); break;
    case 8: hipLaunchKernelGGL(fp8bq::resident_quant<8>, g, b, 0, st, xs, qs, s, p.nchunks, ticks); break;
    case 16: hipLaunchKernelGGL(fp8bq::resident_quant<16>, g, b, 0, st, xs, qs, s, p.nchunks, ticks); break;
    case 32: hipLaunchKernelGGL(fp8bq::resident_quant<32>, g, b, 0, st, xs, qs, s, p.nchunks, ticks); break;
    default:
      hipLaunchKernelGGL(fp8bq::resident_quant<fp8bq::kResMaxLoads>, g, b, 0, st, xs, qs, s, p.nchunks, ticks);
      break;
  }
}

// Several resident tensors: persistent launches of up to kResGroupCap tensors
// over at most `cap` workgroups; tensor i takes the next plan.grid
// workgroups after tensor i-1's (wrapping around).  256 tensors per launch
// against 128: 8 MoE layers (384 tensors each) 66.7% -> 68.2% of peak.

void launch_resident_group(const std::vector<std::pair<const fp8bq_tensor*, ResPlan>>& res, int cap,
                           int tick_mhz, hipStream_t st) {
  const uint64_t ticks = resident_wait_ticks(tick_mhz);
  for (size_t i0 = 0; i0 < res.size(); i0 += kResGroupCap) {
    const size_t c = res.size() - i0 < static_cast<size_t>(kResGroupCap) ? res.size() - i0 : kResGroupCap;
    int64_t want = 0;
    for (size_t i = 0; i < c; ++i) want += res[i0 + i].second.grid;
    const uint32_t g = static_cast<uint32_t>(want < cap ? want : cap);
    fp8bq::ResGroupArgs<kResGroupCap> a;
    std::memset(&a, 0, sizeof(a));
    uint32_t cursor = 0;
    for (size_t i = 0; i < c; ++i) {
      const fp8bq_tensor& t = *res[i0 + i].first;
      const ResPlan& p = res[i0 + i].second;
      fp8bq::ResEntry& e = a.e[i];
      e.x = static_cast<const uint16_t*>(t.x);
      e.q = static_cast<uint8_t*>(t.q);
      e.s = t.scale_inv;
      e.nchunks = p.nchunks;
      e.grid = p.grid;
      e.first = cursor;
      e.loads = p.L;
      cursor = static_cast<uint32_t>((static_cast<uint64_t>(cursor) + p.grid) % g);
    }
    hipLaunchKernelGGL(fp8bq::resident_group<kResGroupCap>, dim3(g), dim3(fp8bq::kThreads), 0, st,
                       a, static_cast<int32_t>(c), ticks);
  }
}

constexpr int kBigGroupCap = 128;  // tensors per grouped large-tile launch

// Whole tensors with large tiles, up to kBigGroupCap per group: 3 launches per
// group (slot maxima, tile scales, quantize).  Returns false if the group's
// counts do not fit 32 bits or a tensor's slots do not fit its q (the caller
// then goes per tensor).
bool launch_big_group(const fp8bq_tensor* const* ts, int32_t n, int32_t bm, int32_t bn,
                      hipStream_t st) {
  fp8bq::BigGroupArgs<kBigGroupCap> a;
  std::memset(&a, 0, sizeof(a));
  int64_t tiles = 0, maxi = 0, quanti = 0;
  for (int32_t i = 0; i < n; ++i) {
    const fp8bq_tensor& t = *ts[i];
    const fp8bq::Big b = make_big(t.x, t.M, t.N, bm, bn, 0, 0, t.q);
    if (!big_slots_fit(b)) return false;
    a.tile_start[i] = static_cast<int32_t>(tiles);
    a.max_start[i] = static_cast<int32_t>(maxi);
    a.quant_start[i] = static_cast<int32_t>(quanti);
    a.e[i].x = static_cast<const uint16_t*>(t.x);
    a.e[i].q = static_cast<uint8_t*>(t.q);
    a.e[i].s = t.scale_inv;
    a.e[i].M = static_cast<int32_t>(t.M);
    a.e[i].N = static_cast<int32_t>(t.N);
    a.e[i].cpt = static_cast<int32_t>(b.cpt);
    a.e[i].flags = b.flat | (b.vec << 1);
    a.e[i].cpm = b.cpm;
    tiles += b.TMl * b.TNl;
    maxi += big_max_items(b);
    quanti += b.items;
    if (tiles > INT32_MAX || maxi > INT32_MAX || quanti > INT32_MAX || b.cpt > INT32_MAX) {
      return false;
    }
  }
  a.tile_start[n] = static_cast<int32_t>(tiles);
  a.max_start[n] = static_cast<int32_t>(maxi);
  a.quant_start[n] = static_cast<int32_t>(quanti);
  const dim3 blk(fp8bq::kThreads);
  hipLaunchKernelGGL((fp8bq::big_group_max<kBigGroupCap>), dim3(grid_for(maxi)), blk, 0, st, a, n,
                     bm, bn);
  hipLaunchKernelGGL((fp8bq::big_group_reduce<kBigGroupCap>), dim3(grid_for(tiles)), blk, 0, st, a,
                     n);
  hipLaunchKernelGGL((fp8bq::big_group_quant<kBigGroupCap>), dim3(grid_for(quanti)), blk, 0, st, a,
                     n, bm, bn);
  return true;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

template <int KIND, int CAP>
void launch_args(const std::vector<Desc>& ds, const std::vector<int64_t>& st, int32_t bm,
                 int32_t bn, int64_t total, hipStream_t s) {
  fp8bq::GroupArgs<CAP> a;
  std::memset(&a, 0, sizeof(a));
  const int32_t n = static_cast<int32_t>(ds.size());
  for (int32_t i = 0; i < n; ++i) {
    a.start[i] = static_cast<int32_t>(st[i]);
    a.t[i].x = ds[i].x;
    a.t[i].q = ds[i].q;
    a.t[i].s = ds[i].s;
    a.t[i].M = static_cast<int32_t>(ds[i].M);
    a.t[i].N = static_cast<int32_t>(ds[i].N);
    a.t[i].body = ds[i].body;
  }
  a.start[n] = static_cast<int32_t>(total);
  if (KIND == fp8bq::kR128 && all_flat(ds)) {
    hipLaunchKernelGGL((fp8bq::quantize_group_args_flat<CAP>), dim3(grid_for(total)),
                       dim3(fp8bq::kThreads), kLds4PerCu, s, a, n, static_cast<int32_t>(total));
    return;
  }
  hipLaunchKernelGGL((fp8bq::quantize_group_args<KIND, CAP>), dim3(grid_for(total)),
                     dim3(fp8bq::kThreads), lds_of(KIND, all_flat(ds), n), s, a, n, bm, bn,
                     static_cast<int32_t>(total));
}

template <int KIND>
void launch_args_kind(const std::vector<Desc>& ds, const std::vector<int64_t>& st, int32_t bm,
                      int32_t bn, int64_t total, hipStream_t s) {
  const size_t n = ds.size();
  if (n <= 8) {
    launch_args<KIND, 8>(ds, st, bm, bn, total, s);
  } else if (n <= 64) {
    launch_args<KIND, 64>(ds, st, bm, bn, total, s);
  } else {
    launch_args<KIND, fp8bq::kArgsMax>(ds, st, bm, bn, total, s);
  }
}

// A table larger than the kernel-argument capacity, without the host-to-device
// copy: one launch per run of at most kArgsMax tensors whose units fit in 32
// bits (a single tensor always does).  Serves calls made under graph capture,
// where a copy from the library's staging memory would be replayed from a
// buffer the library reuses.
template <int KIND>
void launch_args_chunks(const std::vector<Desc>& ds, const std::vector<int64_t>& st, int32_t bm,
                        int32_t bn, int64_t total, hipStream_t s) {
  std::vector<Desc> cd;
  std::vector<int64_t> cs;
  const size_t n = ds.size();
  size_t i = 0;
  while (i < n) {
    cd.clear();
    cs.clear();
    const int64_t base = st[i];
    size_t j = i;
    while (j < n && cd.size() < static_cast<size_t>(fp8bq::kArgsMax)) {
      const int64_t end = j + 1 < n ? st[j + 1] : total;
      if (!cd.empty() && end - base > INT32_MAX) break;
      cd.push_back(ds[j]);
      cs.push_back(st[j] - base);
      ++j;
    }
    const int64_t end = j < n ? st[j] : total;
    launch_args_kind<KIND>(cd, cs, bm, bn, end - base, s);
    i = j;
  }
}

// False only when the stream is known not to be capturing a graph.
bool maybe_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

// Host copies of a grouped call's table, reused per thread.
thread_local std::vector<Desc> g_descs;
thread_local std::vector<int64_t> g_starts;

size_t descs_bytes(int32_t count) { return align_up(sizeof(Desc) * static_cast<size_t>(count), 256); }

// Per device: the address of that device's copy of `scratch`, looked up once
// with the device current (nullptr until then).
std::atomic<unsigned char*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_pointer(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failed(e);
  if (dev < 0 || dev >= kMaxDevices) return FP8BQ_ERR_UNSUPPORTED_DEVICE;
  unsigned char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_failed(e);
      p = static_cast<unsigned char*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8BQ_OK;
}

int quantize_many_impl(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                       unsigned char* workspace, void* stream);

// Host staging of one grouped call's descriptor table, reused per thread.
thread_local std::vector<unsigned char> g_stage;

// Checks one shard call's arguments (QUANT: fp8bq_quantize_amax, else
// fp8bq_tile_amax) before any HIP call and describes the shard in *b.
// *empty is set for M == 0 or N == 0, which is not an error.
int check_shard(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, int32_t row_phase,
                int32_t col_phase, const float* amax, void* q, float* scale_inv, bool quant,
                fp8bq::Big* b, bool* empty) {
  *empty = false;
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX || bm < 1 || bn < 1) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  if (row_phase < 0 || row_phase >= bm || col_phase < 0 || col_phase >= bn) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  if (M == 0 || N == 0) {
    *empty = true;
    return FP8BQ_OK;
  }
  if (x == nullptr || amax == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (quant && (q == nullptr || scale_inv == nullptr)) return FP8BQ_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(x) & 1) != 0 || (reinterpret_cast<uintptr_t>(amax) & 3) != 0 ||
      (quant && (reinterpret_cast<uintptr_t>(scale_inv) & 3) != 0)) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  *b = make_big(x, M, N, bm, bn, row_phase, col_phase, quant ? q : nullptr);
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(N);
  const uint64_t nt = 4 * static_cast<uint64_t>(b->TMl * b->TNl);
  if (!quant) return overlap(x, 2 * n, amax, nt) ? FP8BQ_ERR_INVALID_ARGUMENT : FP8BQ_OK;
  // amax may be scale_inv itself (converted in place), but not partly overlap it.
  const bool same = static_cast<const void*>(amax) == static_cast<const void*>(scale_inv);
  if (overlap(x, 2 * n, q, n) || overlap(x, 2 * n, scale_inv, nt) || overlap(q, n, scale_inv, nt) ||
      overlap(x, 2 * n, amax, nt) || overlap(q, n, amax, nt) ||
      (!same && overlap(amax, nt, scale_inv, nt))) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  return FP8BQ_OK;
}

template <int PASS, bool ROWS>
void launch_shard_group(const fp8bq::ShardGroupArgs<fp8bq::kShardArgsMax>& a, int32_t n,
                        int32_t bm, int32_t bn, int64_t total, unsigned lds, hipStream_t st) {
  hipLaunchKernelGGL((fp8bq::shard_group<PASS, ROWS, fp8bq::kShardArgsMax>), dim3(grid_for(total)),
                     dim3(fp8bq::kThreads), lds, st, a, n, bm, bn, static_cast<int32_t>(total));
}

// Grouped shard calls: every entry is checked first (nothing is enqueued on
// an argument error); entries that take the small-tile kernels go in
// launches of up to kShardArgsMax entries with the table in the kernel
// arguments, the others in their own two-pass launches, all on `stream`.
int shard_many(const fp8bq_shard* list, int32_t count, int32_t bm, int32_t bn, void* stream,
               int pass) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count == 0) return FP8BQ_OK;
  if (list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  thread_local std::vector<fp8bq::Big> bigs;
  thread_local std::vector<int32_t> which;
  bigs.clear();
  which.clear();
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_shard& t = list[i];
    fp8bq::Big b;
    bool empty = false;
    const int st = check_shard(t.x, t.M, t.N, bm, bn, t.row_phase, t.col_phase, t.amax, t.q,
                               t.scale_inv, pass == 1, &b, &empty);
    if (st != FP8BQ_OK) return st;
    if (empty) continue;
    bigs.push_back(b);
    which.push_back(i);
  }
  if (bigs.empty()) return FP8BQ_OK;
  int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool rows = bm == 1 && bn <= 128;
  const unsigned lds =
      pass == 1 && static_cast<int64_t>(bm) * static_cast<int64_t>(bn) >= fp8bq::kRegTile ? kLds4PerCu : 0u;
  fp8bq::ShardGroupArgs<fp8bq::kShardArgsMax> a;
  int32_t n = 0;
  int64_t total = 0;
  // [128,128] quantize passes take four-tile units (shard_group_wide)
  const bool wide = pass == 1 && bm == 128 && bn == 128;
  auto flush = [&]() {
    if (n == 0) return;
    a.start[n] = static_cast<int32_t>(total);
    if (wide) {
      hipLaunchKernelGGL((fp8bq::shard_group_wide<fp8bq::kShardArgsMax>), dim3(grid_for(total)),
                         dim3(fp8bq::kThreads), kLds2PerCu, s, a, n, static_cast<int32_t>(total));
    } else if (pass == 0) {
      if (rows) launch_shard_group<0, true>(a, n, bm, bn, total, lds, s);
      else launch_shard_group<0, false>(a, n, bm, bn, total, lds, s);
    } else {
      if (rows) launch_shard_group<1, true>(a, n, bm, bn, total, lds, s);
      else launch_shard_group<1, false>(a, n, bm, bn, total, lds, s);
    }
    n = 0;
    total = 0;
  };
  for (size_t k = 0; k < bigs.size(); ++k) {
    const fp8bq::Big& b = bigs[k];
    const fp8bq_shard& t = list[which[k]];
    if (!shard_small_ok(b)) {  // large or unaligned tiles: this entry's own launches
      if (pass == 0) {
        launch_big_amax(b, t.amax, s);
      } else {
        launch_big_quant(b, t.amax, t.scale_inv, s);
      }
      continue;
    }
    const int64_t units =
        rows ? ceil_div(b.M, 64) * b.TNl : (wide ? b.TMl * ceil_div(b.TNl, 4) : b.TMl * b.TNl);
    if (n == fp8bq::kShardArgsMax || total + units > INT32_MAX) flush();
    if (units > INT32_MAX) {  // a single entry beyond 32-bit units: its own launch
      launch_shard_small(pass, b, t.amax, pass == 0 ? t.amax : t.scale_inv, s);
      continue;
    }
    fp8bq::ShardEntry& e = a.e[n];
    e.x = b.x;
    e.q = b.q;
    e.amax = t.amax;
    e.out = pass == 0 ? t.amax : t.scale_inv;
    e.M = static_cast<int32_t>(b.M);
    e.N = static_cast<int32_t>(b.N);
    e.row_phase = b.row_phase;
    e.col_phase = b.col_phase;
    a.start[n] = static_cast<int32_t>(total);
    total += units;
    ++n;
  }
  flush();
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

// Checks a dequantization call; *vec says whether it takes the vector body.
// One grouped dequantization launch from a table filled up to entry n:
// copied into a table of CAP entries, with the search's padding (INT32_MAX
// past start[n], and in the coarse entries whose bucket lies past it).
template <int CAP>
void launch_dq_group(const fp8bq::DqGroupArgs<fp8bq::kDqArgsMax>& full, int32_t n, int32_t total,
                     bool f32, dim3 grid, dim3 blk, hipStream_t s) {
  fp8bq::DqGroupArgs<CAP> a;
  std::memset(&a, 0, sizeof(a));
  for (int k = 0; k <= n; ++k) a.start[k] = full.start[k];
  for (int k = n + 1; k < CAP + fp8bq::kDqBucket; ++k) a.start[k] = INT32_MAX;
  for (int k = 0; k < CAP / fp8bq::kDqBucket; ++k) {
    a.coarse[k] = fp8bq::kDqBucket * k <= n ? a.start[fp8bq::kDqBucket * k] : INT32_MAX;
  }
  for (int k = 0; k < n; ++k) a.e[k] = full.e[k];
  if (f32) {
    hipLaunchKernelGGL((fp8bq::dequant_group<fp8bq::kOutF32, CAP>), grid, blk, 0, s, a, n, total);
  } else {
    hipLaunchKernelGGL((fp8bq::dequant_group<fp8bq::kOutBF16, CAP>), grid, blk, 0, s, a, n, total);
  }
}

int check_dequant(const void* q, const float* scale_inv, int64_t M, int64_t N, int32_t bm,
                  int32_t bn, void* out, int32_t out_dtype, bool* vec) {
  *vec = false;
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX || bm < 1 || bn < 1) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  if (out_dtype != FP8BQ_OUT_F32 && out_dtype != FP8BQ_OUT_BF16) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (M == 0 || N == 0) return FP8BQ_OK;
  if (q == nullptr || scale_inv == nullptr || out == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  const uintptr_t qa = reinterpret_cast<uintptr_t>(q);
  const uintptr_t sa = reinterpret_cast<uintptr_t>(scale_inv);
  const uintptr_t oa = reinterpret_cast<uintptr_t>(out);
  const uint64_t esize = out_dtype == FP8BQ_OUT_F32 ? 4 : 2;
  if ((sa & 3) != 0 || (oa & (esize - 1)) != 0) return FP8BQ_ERR_INVALID_ARGUMENT;
  const int64_t TM = ceil_div(M, bm);
  const int64_t TN = ceil_div(N, bn);
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(N);
  const uint64_t ns = static_cast<uint64_t>(TM) * static_cast<uint64_t>(TN);
  if (overlap(out, esize * n, q, n) || overlap(out, esize * n, scale_inv, 4 * ns)) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  const int64_t G = out_dtype == FP8BQ_OUT_F32 ? 4 : 8;
  *vec = (N % G) == 0 && (bn % G) == 0 && (qa % G) == 0 && (oa & 15) == 0;
  return FP8BQ_OK;
}

void launch_dequant_vec(const void* q, const float* scale_inv, int64_t M, int64_t N, int32_t bm,
                        int32_t bn, void* out, int32_t out_dtype, hipStream_t s) {
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const int32_t tn = static_cast<int32_t>(ceil_div(N, bn));
  const int64_t G = out_dtype == FP8BQ_OUT_F32 ? 4 : 8;
  const int64_t groups = M * N / G;
  const int64_t per_block = static_cast<int64_t>(fp8bq::kThreads) * fp8bq::kDqUnroll;
  const unsigned grid = grid_for((groups + per_block - 1) / per_block);
  const int64_t gpr = N / G;  // groups per row, < 2^29
  const int64_t stride = static_cast<int64_t>(grid) * per_block;
  const fp8bq::Div31 by_gpr = fp8bq::make_div31(static_cast<uint32_t>(gpr));
  const fp8bq::Div31 by_bm = fp8bq::make_div31(static_cast<uint32_t>(bm));
  const fp8bq::Div31 by_bn = fp8bq::make_div31(static_cast<uint32_t>(bn));
  const int64_t step_rows = stride / gpr;
  const int32_t step_cols = static_cast<int32_t>(stride % gpr);
  if (out_dtype == FP8BQ_OUT_F32) {
    hipLaunchKernelGGL(fp8bq::dequant_vec<fp8bq::kOutF32>, dim3(grid), dim3(fp8bq::kThreads), 0, s,
                       qb, scale_inv, static_cast<int32_t>(gpr), tn, by_gpr, by_bm, by_bn, out,
                       groups, static_cast<int32_t>(M - 1), step_rows, step_cols);
  } else {
    hipLaunchKernelGGL(fp8bq::dequant_vec<fp8bq::kOutBF16>, dim3(grid), dim3(fp8bq::kThreads), 0, s,
                       qb, scale_inv, static_cast<int32_t>(gpr), tn, by_gpr, by_bm, by_bn, out,
                       groups, static_cast<int32_t>(M - 1), step_rows, step_cols);
  }
}

void launch_dequant_elem(const void* q, const float* scale_inv, int64_t M, int64_t N, int32_t bm,
                         int32_t bn, void* out, int32_t out_dtype, hipStream_t s) {
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const int32_t tn = static_cast<int32_t>(ceil_div(N, bn));
  const int64_t n = M * N;
  const int64_t blocks = (n + fp8bq::kThreads - 1) / fp8bq::kThreads;
  const dim3 grid(static_cast<unsigned>(blocks < 65536 * 16 ? blocks : 65536 * 16));
  if (out_dtype == FP8BQ_OUT_F32) {
    hipLaunchKernelGGL(fp8bq::dequant_elem<fp8bq::kOutF32>, grid, dim3(fp8bq::kThreads), 0, s, qb,
                       scale_inv, N, bm, bn, tn, out, n);
  } else {
    hipLaunchKernelGGL(fp8bq::dequant_elem<fp8bq::kOutBF16>, grid, dim3(fp8bq::kThreads), 0, s, qb,
                       scale_inv, N, bm, bn, tn, out, n);
  }
}

}  // namespace

extern "C" {

int fp8bq_quantize(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, void* q,
                   float* scale_inv, void* stream) {
  if (bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  int kind = kind_of(bm, bn);
  if (kind == fp8bq::kT128 || kind == fp8bq::kT64) {
    kind = wide_kind(kind, wide_units(x, M, N, q, kind == fp8bq::kT128 ? 128 : 64));
  }
  Desc d;
  int64_t units = 0;
  int st = make_desc(x, M, N, bm, bn, q, scale_inv, kind, &d, &units);
  if (st != FP8BQ_OK || units == 0) return st;
  st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (big_tiles(M, N, bm, bn)) {
    int tick_mhz = 0;
    ResPlan p;
    if (resident_plan(x, M, N, bm, bn, q, resident_capacity(&tick_mhz), &p)) {
      const fp8bq::ResTensor t{static_cast<uint8_t*>(q), scale_inv};
      launch_resident_prep(&t, 1, s);
      launch_resident(p, x, q, scale_inv, tick_mhz, s);
    } else {
      launch_big_tensor(make_big(x, M, N, bm, bn, 0, 0, q), scale_inv, s);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
  }
  switch (d.body != fp8bq::kBodyVec && d.body != fp8bq::kBodyFlat ? static_cast<int>(fp8bq::kGeneral) : kind) {
    case fp8bq::kT128: launch_one<fp8bq::kT128>(d, bm, bn, units, s); break;
    case fp8bq::kT128W: launch_one<fp8bq::kT128W>(d, bm, bn, units, s); break;
    case fp8bq::kT64W: launch_one<fp8bq::kT64W>(d, bm, bn, units, s); break;
    case fp8bq::kT64: launch_one<fp8bq::kT64>(d, bm, bn, units, s); break;
    case fp8bq::kR128: launch_one<fp8bq::kR128>(d, bm, bn, units, s); break;
    default: launch_one<fp8bq::kGeneral>(d, bm, bn, units, s); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

size_t fp8bq_many_workspace_bytes(int32_t count) {
  if (count <= fp8bq::kArgsMax) return 0;  // the table travels in the kernel arguments
  return descs_bytes(count) + align_up(sizeof(int64_t) * (static_cast<size_t>(count) + 1), 256);
}

int fp8bq_quantize_many(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count == 0) return FP8BQ_OK;
  if (list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  const size_t need = fp8bq_many_workspace_bytes(count);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)) {
    return FP8BQ_ERR_WORKSPACE;
  }
  return quantize_many_impl(list, count, bm, bn, static_cast<unsigned char*>(workspace), stream);
}

int fp8bq_quantize_many_noalloc(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                                void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count == 0) return FP8BQ_OK;
  if (list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count > FP8BQ_NOALLOC_MAX_TENSORS) return FP8BQ_ERR_WORKSPACE;
  return quantize_many_impl(list, count, bm, bn, nullptr, stream);
}

}  // extern "C"

namespace {

// The body of both grouped entry points.  `workspace` receives the
// descriptor table when it travels by copy; nullptr selects this device's
// copy of `scratch` instead (fp8bq_quantize_many_noalloc; its count is
// already bounded by FP8BQ_NOALLOC_MAX_TENSORS).  Every argument check runs
// before the first HIP call.
int quantize_many_impl(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                       unsigned char* workspace, void* stream) {
  const size_t need = fp8bq_many_workspace_bytes(count);
  int kind = kind_of(bm, bn);
  if (kind == fp8bq::kT128 || kind == fp8bq::kT64) {
    const int64_t rows = kind == fp8bq::kT128 ? 128 : 64;
    int64_t wide = 0;
    for (int32_t i = 0; i < count && wide >= 0; ++i) {
      const int64_t w = wide_units(list[i].x, list[i].M, list[i].N, list[i].q, rows);
      wide = w < 0 ? -1 : wide + w;
    }
    kind = wide_kind(kind, wide);
  }
  g_descs.clear();
  g_starts.clear();
  int64_t total = 0;
  bool any_big = false;
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_tensor& t = list[i];
    int64_t units = 0;
    Desc d;
    const int st = make_desc(t.x, t.M, t.N, bm, bn, t.q, t.scale_inv, kind, &d, &units);
    if (st != FP8BQ_OK) return st;
    if (units == 0) continue;
    if (big_tiles(t.M, t.N, bm, bn)) {  // two-pass path, launched per tensor below
      any_big = true;
      continue;
    }
    g_descs.push_back(d);
    g_starts.push_back(total);
    total += units;
  }
  const int32_t n = static_cast<int32_t>(g_descs.size());
  if (n == 0 && !any_big) return FP8BQ_OK;
  // The table in the kernel arguments indexes units with 32 bits.
  const bool args_fit = n <= fp8bq::kArgsMax && total <= INT32_MAX;
  int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (any_big) {
    // Whole tensors that fit in registers: a preparation launch for all of
    // them, then persistent resident launches.
    int tick_mhz = 0;
    const int cap = resident_capacity(&tick_mhz);
    std::vector<std::pair<const fp8bq_tensor*, ResPlan>> res;
    std::vector<fp8bq::ResTensor> res_t;
    for (int32_t i = 0; i < count; ++i) {
      const fp8bq_tensor& t = list[i];
      ResPlan p;
      if (t.M == 0 || t.N == 0 || !big_tiles(t.M, t.N, bm, bn) ||
          !resident_plan(t.x, t.M, t.N, bm, bn, t.q, cap, &p)) {
        continue;
      }
      res.emplace_back(&t, p);
      res_t.push_back(fp8bq::ResTensor{static_cast<uint8_t*>(t.q), t.scale_inv});
    }
    if (!res.empty()) {
      if (res.size() > 1) {
        // Side by side in a persistent launch, the fewest workgroups per
        // tensor (48 chunks per thread) measured best: dense set 66.7% ->
        // 68.6% of peak, one layer 64.5% -> 69.4%, 8 MoE layers 52.6% ->
        // 66.4% (32 chunks: 67.3 / 67.8 / 64.8%; 16: 62.7 / 59.3 / 54.5%).
        for (auto& r : res) {
          const int64_t g = ceil_div(r.second.nchunks, int64_t{fp8bq::kThreads} * fp8bq::kResMaxLoads);
          r.second.L = fp8bq::kResMaxLoads;
          r.second.grid = static_cast<uint32_t>(g);
        }
      }
      launch_resident_prep(res_t.data(), static_cast<int>(res_t.size()), s);
      if (res.size() == 1) {
        launch_resident(res[0].second, res[0].first->x, res[0].first->q, res[0].first->scale_inv,
                        tick_mhz, s);
      } else {
        launch_resident_group(res, cap, tick_mhz, s);
      }
    }
    // The other large-tile tensors: grouped two-pass launches, kBigGroupCap
    // tensors at a time.
    std::vector<const fp8bq_tensor*> group;
    auto flush = [&]() {
      if (group.empty()) return;
      if (!launch_big_group(group.data(), static_cast<int32_t>(group.size()), bm, bn, s)) {
        for (const fp8bq_tensor* t : group) {  // counts beyond 32 bits: per tensor
          launch_big_tensor(make_big(t->x, t->M, t->N, bm, bn, 0, 0, t->q), t->scale_inv, s);
        }
      }
      group.clear();
    };
    for (int32_t i = 0; i < count; ++i) {
      const fp8bq_tensor& t = list[i];
      ResPlan p;
      if (t.M == 0 || t.N == 0 || !big_tiles(t.M, t.N, bm, bn) ||
          resident_plan(t.x, t.M, t.N, bm, bn, t.q, cap, &p)) {
        continue;
      }
      group.push_back(&t);
      if (static_cast<int>(group.size()) == kBigGroupCap) flush();
    }
    flush();
  }
  if (n > 0 && args_fit) {
    // The table travels in the kernel arguments: no copy, no workspace.
    switch (kind) {
      case fp8bq::kT128: launch_args_kind<fp8bq::kT128>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT128W: launch_args_kind<fp8bq::kT128W>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT64W: launch_args_kind<fp8bq::kT64W>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT64: launch_args_kind<fp8bq::kT64>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kR128: launch_args_kind<fp8bq::kR128>(g_descs, g_starts, bm, bn, total, s); break;
      default: launch_args_kind<fp8bq::kGeneral>(g_descs, g_starts, bm, bn, total, s); break;
    }
  } else if (n > 0 && need == 0) {
    // At most kArgsMax tensors but more than 2^31 units in all (tiny blocks):
    // one launch per tensor.
    for (int32_t i = 0; i < n; ++i) {
      const Desc& d = g_descs[i];
      const int64_t units = (i + 1 < n ? g_starts[i + 1] : total) - g_starts[i];
      switch (d.body != fp8bq::kBodyVec && d.body != fp8bq::kBodyFlat ? static_cast<int>(fp8bq::kGeneral) : kind) {
        case fp8bq::kT128: launch_one<fp8bq::kT128>(d, bm, bn, units, s); break;
        case fp8bq::kT128W: launch_one<fp8bq::kT128W>(d, bm, bn, units, s); break;
        case fp8bq::kT64W: launch_one<fp8bq::kT64W>(d, bm, bn, units, s); break;
        case fp8bq::kT64: launch_one<fp8bq::kT64>(d, bm, bn, units, s); break;
        case fp8bq::kR128: launch_one<fp8bq::kR128>(d, bm, bn, units, s); break;
        default: launch_one<fp8bq::kGeneral>(d, bm, bn, units, s); break;
      }
    }
  } else if (n > 0 && maybe_capturing(s)) {
    // Under graph capture: several launches with the table in their arguments.
    switch (kind) {
      case fp8bq::kT128: launch_args_chunks<fp8bq::kT128>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT128W: launch_args_chunks<fp8bq::kT128W>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT64W: launch_args_chunks<fp8bq::kT64W>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kT64: launch_args_chunks<fp8bq::kT64>(g_descs, g_starts, bm, bn, total, s); break;
      case fp8bq::kR128: launch_args_chunks<fp8bq::kR128>(g_descs, g_starts, bm, bn, total, s); break;
      default: launch_args_chunks<fp8bq::kGeneral>(g_descs, g_starts, bm, bn, total, s); break;
    }
  } else if (n > 0) {
    // Larger groups: the table is copied into the workspace on the stream.
    g_stage.resize(need);
    std::memcpy(g_stage.data(), g_descs.data(), sizeof(Desc) * static_cast<size_t>(n));
    int64_t* start = reinterpret_cast<int64_t*>(g_stage.data() + descs_bytes(count));
    std::memcpy(start, g_starts.data(), sizeof(int64_t) * static_cast<size_t>(n));
    start[n] = total;
    unsigned char* ws = workspace;
    if (ws == nullptr) {
      st = scratch_pointer(&ws);
      if (st != FP8BQ_OK) return st;
    }
    const size_t used = descs_bytes(count) + sizeof(int64_t) * (static_cast<size_t>(n) + 1);
    hipError_t e = hipMemcpyAsync(ws, g_stage.data(), used, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_failed(e);
    const unsigned lds = lds_of(kind, all_flat(g_descs), n);
    const Desc* d_descs = reinterpret_cast<const Desc*>(ws);
    const int64_t* d_start = reinterpret_cast<const int64_t*>(ws + descs_bytes(count));
    switch (kind) {
      case fp8bq::kT128: launch_group<fp8bq::kT128>(d_descs, d_start, n, bm, bn, total, lds, s); break;
      case fp8bq::kT128W: launch_group<fp8bq::kT128W>(d_descs, d_start, n, bm, bn, total, lds, s); break;
      case fp8bq::kT64W: launch_group<fp8bq::kT64W>(d_descs, d_start, n, bm, bn, total, lds, s); break;
      case fp8bq::kT64: launch_group<fp8bq::kT64>(d_descs, d_start, n, bm, bn, total, lds, s); break;
      case fp8bq::kR128: launch_group<fp8bq::kR128>(d_descs, d_start, n, bm, bn, total, lds, s); break;
      default: launch_group<fp8bq::kGeneral>(d_descs, d_start, n, bm, bn, total, lds, s); break;
    }
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

// Rows of a row shard: the first `top` rows share a tile row with the
// shards above, the last `bottom` rows one with the shards below; the rows
// between are whole tile rows of this shard alone.
struct RowParts {
  int64_t top = 0;
  int64_t bottom = 0;
  int64_t TMl = 0;  // local tile rows
  int64_t TN = 0;   // tile columns
};

int row_parts(int64_t M, int32_t bm, int32_t row_phase, RowParts* p) {
  if (M < 0 || M > INT32_MAX || bm < 1 || row_phase < 0 || row_phase >= bm) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  p->top = std::min<int64_t>(M, (bm - row_phase) % bm);
  p->bottom = (M - p->top) % bm;
  p->TMl = ceil_div(row_phase + M, bm);
  return FP8BQ_OK;
}

// Checks one row-shard entry as a whole: ranges, pointers, alignment and
// the overlaps of x, q, scale_inv and the two edge maxima (each edge's
// maxima may be its own scale row, converted in place).  Fills *p.
int check_row_shard(const fp8bq_row_shard& r, int32_t bm, int32_t bn, RowParts* p) {
  int st = row_parts(r.M, bm, r.row_phase, p);
  if (st != FP8BQ_OK || r.N < 0 || r.N > INT32_MAX || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  p->TN = ceil_div(r.N, bn);
  if (r.M == 0 || r.N == 0) return FP8BQ_OK;
  if (r.x == nullptr || r.q == nullptr || r.scale_inv == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(r.x) & 1) != 0 || (reinterpret_cast<uintptr_t>(r.scale_inv) & 3) != 0) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  const uint64_t n = static_cast<uint64_t>(r.M) * static_cast<uint64_t>(r.N);
  const uint64_t ns = 4 * static_cast<uint64_t>(p->TMl) * static_cast<uint64_t>(p->TN);
  const uint64_t na = 4 * static_cast<uint64_t>(p->TN);
  if (overlap(r.x, 2 * n, r.q, n) || overlap(r.x, 2 * n, r.scale_inv, ns) || overlap(r.q, n, r.scale_inv, ns)) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  const float* rows[2] = {r.scale_inv, r.scale_inv + (p->TMl - 1) * p->TN};  // first, last scale row
  const float* am[2] = {r.top_amax, r.bottom_amax};
  const bool used[2] = {p->top > 0, p->bottom > 0};
  for (int k = 0; k < 2; ++k) {
    if (!used[k]) continue;
    if (am[k] == nullptr || (reinterpret_cast<uintptr_t>(am[k]) & 3) != 0) return FP8BQ_ERR_INVALID_ARGUMENT;
    if (overlap(am[k], na, r.x, 2 * n) || overlap(am[k], na, r.q, n) ||
        (am[k] != rows[k] && overlap(am[k], na, r.scale_inv, ns))) {
      return FP8BQ_ERR_INVALID_ARGUMENT;
    }
  }
  if (used[0] && used[1] && overlap(am[0], na, am[1], na)) return FP8BQ_ERR_INVALID_ARGUMENT;
  return FP8BQ_OK;
}

// Host lists of a row-shard call, reused per thread.
thread_local std::vector<fp8bq_shard> g_row_edges;
thread_local std::vector<fp8bq_tensor> g_row_inner;

// The edge slabs of every entry as shard entries: pass 0 writes their
// partial maxima to top_amax / bottom_amax, pass 1 quantizes them with
// those maxima into their q rows and first / last scale row.
void row_edges(const fp8bq_row_shard* list, int32_t count, int32_t bm, int32_t bn, int pass) {
  g_row_edges.clear();
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_row_shard& r = list[i];
    RowParts p;
    (void)check_row_shard(r, bm, bn, &p);  // already checked: fills p
    if (r.M == 0 || r.N == 0) continue;
    const bool quant = pass == 1;
    if (p.top > 0) {
      g_row_edges.push_back(fp8bq_shard{r.x, quant ? r.q : nullptr, r.top_amax,
                                        quant ? r.scale_inv : nullptr, p.top, r.N, r.row_phase, 0});
    }
    if (p.bottom > 0) {
      const int64_t r0 = r.M - p.bottom;
      g_row_edges.push_back(fp8bq_shard{
          static_cast<const uint16_t*>(r.x) + r0 * r.N,
          quant ? static_cast<void*>(static_cast<uint8_t*>(r.q) + r0 * r.N) : nullptr, r.bottom_amax,
          quant ? r.scale_inv + (p.TMl - 1) * p.TN : nullptr, p.bottom, r.N, 0, 0});
    }
  }
}

// The edge slabs through the grouped shard calls, in lists of at most
// INT32_MAX entries.
int run_row_edges(int32_t bm, int32_t bn, void* stream, int pass) {
  const size_t n = g_row_edges.size();
  for (size_t i = 0; i < n; i += INT32_MAX) {
    const int32_t c = static_cast<int32_t>(std::min<size_t>(n - i, INT32_MAX));
    const int st = shard_many(g_row_edges.data() + i, c, bm, bn, stream, pass);
    if (st != FP8BQ_OK) return st;
  }
  return FP8BQ_OK;
}

}  // namespace

extern "C" {

int fp8bq_tile_amax(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, int32_t row_phase,
                    int32_t col_phase, float* amax, void* stream) {
  fp8bq::Big b;
  bool empty = false;
  int st = check_shard(x, M, N, bm, bn, row_phase, col_phase, amax, nullptr, nullptr, false, &b,
                       &empty);
  if (st != FP8BQ_OK || empty) return st;
  st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (shard_small_ok(b)) {
    launch_shard_small(0, b, nullptr, amax, s);
  } else {
    launch_big_amax(b, amax, s);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

int fp8bq_quantize_amax(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn,
                        int32_t row_phase, int32_t col_phase, const float* amax, void* q,
                        float* scale_inv, void* stream) {
  fp8bq::Big b;
  bool empty = false;
  int st = check_shard(x, M, N, bm, bn, row_phase, col_phase, amax, q, scale_inv, true, &b, &empty);
  if (st != FP8BQ_OK || empty) return st;
  st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (shard_small_ok(b)) {
    launch_shard_small(1, b, amax, scale_inv, s);
  } else {
    launch_big_quant(b, amax, scale_inv, s);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

int fp8bq_tile_amax_many(const fp8bq_shard* list, int32_t count, int32_t bm, int32_t bn,
                         void* stream) {
  return shard_many(list, count, bm, bn, stream, 0);
}

int fp8bq_quantize_amax_many(const fp8bq_shard* list, int32_t count, int32_t bm, int32_t bn,
                             void* stream) {
  return shard_many(list, count, bm, bn, stream, 1);
}

int fp8bq_row_shard_edges(int64_t M, int32_t bm, int32_t row_phase, int64_t* top, int64_t* bottom) {
  RowParts p;
  if (top == nullptr || bottom == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  const int st = row_parts(M, bm, row_phase, &p);
  if (st != FP8BQ_OK) return st;
  *top = p.top;
  *bottom = p.bottom;
  return FP8BQ_OK;
}

int fp8bq_row_shards_begin(const fp8bq_row_shard* list, int32_t count, int32_t bm, int32_t bn,
                           void* workspace, size_t workspace_bytes, void* maxima_event,
                           void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count > 0 && list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  g_row_inner.clear();
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_row_shard& r = list[i];
    RowParts p;
    const int st = check_row_shard(r, bm, bn, &p);
    if (st != FP8BQ_OK) return st;
    const int64_t inner = r.M - p.top - p.bottom;
    if (r.N == 0 || inner == 0) continue;
    g_row_inner.push_back(fp8bq_tensor{static_cast<const uint16_t*>(r.x) + p.top * r.N,
                                       static_cast<uint8_t*>(r.q) + p.top * r.N,
                                       r.scale_inv + (p.top > 0 ? p.TN : 0), inner, r.N});
  }
  const int32_t n_inner = static_cast<int32_t>(g_row_inner.size());
  const size_t need = fp8bq_many_workspace_bytes(n_inner);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)) {
    return FP8BQ_ERR_WORKSPACE;
  }
  // 1. partial maxima of the edge rows, then the event the exchange waits for
  row_edges(list, count, bm, bn, 0);
  int st = run_row_edges(bm, bn, stream, 0);
  if (st != FP8BQ_OK) return st;
  if (maxima_event != nullptr) {
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(maxima_event), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_failed(e);
  }
  // 2. the whole tile rows between the edges, in one pass
  if (n_inner == 0) return FP8BQ_OK;
  return quantize_many_impl(g_row_inner.data(), n_inner, bm, bn, static_cast<unsigned char*>(workspace),
                            stream);
}

int fp8bq_row_shards_finish(const fp8bq_row_shard* list, int32_t count, int32_t bm, int32_t bn,
                            void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count > 0 && list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < count; ++i) {
    RowParts p;
    const int st = check_row_shard(list[i], bm, bn, &p);
    if (st != FP8BQ_OK) return st;
  }
  row_edges(list, count, bm, bn, 1);
  return run_row_edges(bm, bn, stream, 1);
}

int fp8bq_encode_e4m3(const float* y, void* q, int64_t n, void* stream) {
  if (n < 0) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (n == 0) return FP8BQ_OK;
  if (y == nullptr || q == nullptr || (reinterpret_cast<uintptr_t>(y) & 3) != 0) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  if (overlap(y, 4 * static_cast<uint64_t>(n), q, static_cast<uint64_t>(n))) {
    return FP8BQ_ERR_INVALID_ARGUMENT;
  }
  int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t blocks = (n + fp8bq::kThreads - 1) / fp8bq::kThreads;
  const unsigned grid = static_cast<unsigned>(blocks < 65536 * 16 ? blocks : 65536 * 16);
  hipLaunchKernelGGL(fp8bq::encode_e4m3, dim3(grid), dim3(fp8bq::kThreads), 0, s, y,
                     static_cast<uint8_t*>(q), n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

int fp8bq_dequantize(const void* q, const float* scale_inv, int64_t M, int64_t N, int32_t bm,
                     int32_t bn, void* out, int32_t out_dtype, void* stream) {
  bool vec = false;
  const int st0 = check_dequant(q, scale_inv, M, N, bm, bn, out, out_dtype, &vec);
  if (st0 != FP8BQ_OK || M == 0 || N == 0) return st0;
  const int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (vec) {
    launch_dequant_vec(q, scale_inv, M, N, bm, bn, out, out_dtype, s);
  } else {
    launch_dequant_elem(q, scale_inv, M, N, bm, bn, out, out_dtype, s);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

int fp8bq_dequantize_many(const fp8bq_dq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                          int32_t out_dtype, void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != FP8BQ_OUT_F32 && out_dtype != FP8BQ_OUT_BF16) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count == 0) return FP8BQ_OK;
  if (list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  std::vector<char> vec(static_cast<size_t>(count), 0);
  bool any = false;
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_dq_tensor& t = list[i];
    bool v = false;
    const int st = check_dequant(t.q, t.scale_inv, t.M, t.N, bm, bn, t.out, out_dtype, &v);
    if (st != FP8BQ_OK) return st;
    vec[static_cast<size_t>(i)] = v ? 1 : 0;
    any = any || (t.M > 0 && t.N > 0);
  }
  if (!any) return FP8BQ_OK;
  const int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t G = out_dtype == FP8BQ_OUT_F32 ? 4 : 8;
  const int64_t per_block = static_cast<int64_t>(fp8bq::kThreads) * fp8bq::kDqUnroll;
  const bool f32 = out_dtype == FP8BQ_OUT_F32;
  constexpr int C = fp8bq::kDqArgsMax;
  fp8bq::DqGroupArgs<C> a;
  int32_t n = 0;
  int64_t total = 0;
  auto flush = [&]() {
    if (n == 0) return;
    a.start[n] = static_cast<int32_t>(total);
    const dim3 grid(grid_for(total)), blk(fp8bq::kThreads);
    const int32_t tot = static_cast<int32_t>(total);
    if (n <= fp8bq::kDqBucket) {
      launch_dq_group<fp8bq::kDqBucket>(a, n, tot, f32, grid, blk, s);
    } else {
      launch_dq_group<C>(a, n, tot, f32, grid, blk, s);
    }
    n = 0;
    total = 0;
  };
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_dq_tensor& t = list[i];
    if (t.M == 0 || t.N == 0) continue;
    if (!vec[static_cast<size_t>(i)]) {
      launch_dequant_elem(t.q, t.scale_inv, t.M, t.N, bm, bn, t.out, out_dtype, s);
      continue;
    }
    const int64_t groups = t.M * t.N / G;
    const int64_t runs = ceil_div(groups, per_block);
    if (groups >= (int64_t{1} << 31) - per_block) {  // beyond 32-bit group numbers: its own launch
      launch_dequant_vec(t.q, t.scale_inv, t.M, t.N, bm, bn, t.out, out_dtype, s);
      continue;
    }
    if (n == fp8bq::kDqArgsMax || total + runs > INT32_MAX) flush();
    if (n == 0) std::memset(&a, 0, sizeof(a));
    fp8bq::DqEntry& e = a.e[n];
    e.q = static_cast<const uint8_t*>(t.q);
    e.s = t.scale_inv;
    e.out = t.out;
    e.groups = groups;
    e.gpr = static_cast<int32_t>(t.N / G);
    e.TN = static_cast<int32_t>(ceil_div(t.N, bn));
    e.last_row = static_cast<int32_t>(t.M - 1);
    e.step_rows = static_cast<int32_t>(per_block / (t.N / G));
    e.step_cols = static_cast<int32_t>(per_block % (t.N / G));
    e.by_gpr = fp8bq::make_div31(static_cast<uint32_t>(t.N / G));
    e.by_bm = fp8bq::make_div31(static_cast<uint32_t>(bm));
    e.by_bn = fp8bq::make_div31(static_cast<uint32_t>(bn));
    a.start[n] = static_cast<int32_t>(total);
    total += runs;
    ++n;
  }
  flush();
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

int fp8bq_set_resident_wait_us(int64_t microseconds) {
  if (microseconds < 0 || microseconds > (int64_t{1} << 40)) return FP8BQ_ERR_INVALID_ARGUMENT;
  g_res_wait_us.store(microseconds, std::memory_order_relaxed);
  return FP8BQ_OK;
}

const char* fp8bq_status_string(int status) {
  switch (status) {
    case FP8BQ_OK: return "ok";
    case FP8BQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FP8BQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case FP8BQ_ERR_WORKSPACE: return "workspace null, too small or misaligned";
    case FP8BQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int fp8bq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
