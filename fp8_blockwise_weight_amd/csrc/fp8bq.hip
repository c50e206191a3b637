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
#include <vector>

#include "fp8bq.h"
#include "kernels.hpp"

namespace {

using fp8bq::Desc;

thread_local int g_last_hip_error = 0;

int hip_failed(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return FP8BQ_ERR_HIP;
}

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxUnits = INT32_MAX;  // work units per tensor (32-bit unit math)
constexpr int64_t kMaxGrid = INT32_MAX;   // workgroups per launch

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
  const bool vec = kind != fp8bq::kGeneral && (N % 8) == 0 && (xa & 15) == 0 && (qa & 7) == 0;
  d->x = static_cast<const uint16_t*>(x);
  d->q = static_cast<uint8_t*>(q);
  d->s = s;
  d->M = M;
  d->N = N;
  d->TN = static_cast<int32_t>(TN);
  d->pad = 0;
  d->reserved = 0;
  int64_t u;
  if (vec) {
    const int64_t rows = kind == fp8bq::kT128 ? 128 : 64;
    d->UN = static_cast<int32_t>(ceil_div(N, 128));
    d->general = 0;
    u = ceil_div(M, rows) * d->UN;
  } else {
    if (TN > INT32_MAX) return FP8BQ_ERR_INVALID_ARGUMENT;
    d->UN = static_cast<int32_t>(TN);
    d->general = 1;
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

template <int KIND>
void launch_one(const Desc& d, int32_t bm, int32_t bn, int64_t units, hipStream_t st) {
  hipLaunchKernelGGL(fp8bq::quantize_one<KIND>, dim3(grid_for(units)), dim3(fp8bq::kThreads), 0,
                     st, d, bm, bn, units);
}

template <int KIND>
void launch_group(const Desc* descs, const int64_t* start, int32_t count, int32_t bm, int32_t bn,
                  int64_t units, hipStream_t st) {
  hipLaunchKernelGGL(fp8bq::quantize_group<KIND>, dim3(grid_for(units)), dim3(fp8bq::kThreads), 0,
                     st, descs, start, count, bm, bn, units);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t descs_bytes(int32_t count) { return align_up(sizeof(Desc) * static_cast<size_t>(count), 256); }

// Host staging of one grouped call's descriptor table, reused per thread.
thread_local std::vector<unsigned char> g_stage;

}  // namespace

extern "C" {

int fp8bq_quantize(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, void* q,
                   float* scale_inv, void* stream) {
  if (bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  const int kind = kind_of(bm, bn);
  Desc d;
  int64_t units = 0;
  int st = make_desc(x, M, N, bm, bn, q, scale_inv, kind, &d, &units);
  if (st != FP8BQ_OK || units == 0) return st;
  st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (d.general ? static_cast<int>(fp8bq::kGeneral) : kind) {
    case fp8bq::kT128: launch_one<fp8bq::kT128>(d, bm, bn, units, s); break;
    case fp8bq::kT64: launch_one<fp8bq::kT64>(d, bm, bn, units, s); break;
    case fp8bq::kR128: launch_one<fp8bq::kR128>(d, bm, bn, units, s); break;
    default: launch_one<fp8bq::kGeneral>(d, bm, bn, units, s); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
}

size_t fp8bq_many_workspace_bytes(int32_t count) {
  if (count <= 0) return 0;
  return descs_bytes(count) + align_up(sizeof(int64_t) * (static_cast<size_t>(count) + 1), 256);
}

int fp8bq_quantize_many(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 0 || bm < 1 || bn < 1) return FP8BQ_ERR_INVALID_ARGUMENT;
  if (count == 0) return FP8BQ_OK;
  if (list == nullptr) return FP8BQ_ERR_INVALID_ARGUMENT;
  const size_t need = fp8bq_many_workspace_bytes(count);
  if (workspace == nullptr || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 15) != 0) {
    return FP8BQ_ERR_WORKSPACE;
  }
  const int kind = kind_of(bm, bn);
  g_stage.resize(need);
  Desc* descs = reinterpret_cast<Desc*>(g_stage.data());
  int64_t* start = reinterpret_cast<int64_t*>(g_stage.data() + descs_bytes(count));
  int32_t n = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const fp8bq_tensor& t = list[i];
    int64_t units = 0;
    const int st = make_desc(t.x, t.M, t.N, bm, bn, t.q, t.scale_inv, kind, &descs[n], &units);
    if (st != FP8BQ_OK) return st;
    if (units == 0) continue;
    start[n] = total;
    total += units;
    ++n;
  }
  if (n == 0) return FP8BQ_OK;
  start[n] = total;
  int st = device_check();
  if (st != FP8BQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // The two tables are packed at the front of the workspace in the same
  // layout as the staging buffer, so one copy moves both.
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const size_t used = descs_bytes(count) + sizeof(int64_t) * (static_cast<size_t>(n) + 1);
  hipError_t e = hipMemcpyAsync(ws, g_stage.data(), used, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_failed(e);
  const Desc* d_descs = reinterpret_cast<const Desc*>(ws);
  const int64_t* d_start = reinterpret_cast<const int64_t*>(ws + descs_bytes(count));
  switch (kind) {
    case fp8bq::kT128: launch_group<fp8bq::kT128>(d_descs, d_start, n, bm, bn, total, s); break;
    case fp8bq::kT64: launch_group<fp8bq::kT64>(d_descs, d_start, n, bm, bn, total, s); break;
    case fp8bq::kR128: launch_group<fp8bq::kR128>(d_descs, d_start, n, bm, bn, total, s); break;
    default: launch_group<fp8bq::kGeneral>(d_descs, d_start, n, bm, bn, total, s); break;
  }
  e = hipGetLastError();
  return e == hipSuccess ? FP8BQ_OK : hip_failed(e);
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
