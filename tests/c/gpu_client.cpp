// A native client of libfp8bq on the GPU, with no Python and no torch.
// It reads a BF16 matrix from a file and, on a stream of its own:
//   1. quantizes it with fp8bq_quantize;
//   2. captures fp8bq_quantize_many (one entry, other outputs) in a HIP
//      graph and replays it twice, refilling those outputs with a pattern
//      before each replay (eagerly, outside the graph);
//   3. dequantizes the result of step 1 to fp32 with fp8bq_dequantize, and
//      both results again with one fp8bq_dequantize_many call.
// It checks that both quantizations, and all three dequantizations, agree
// byte for byte and writes
// <prefix>.q (uint8 [M, N]), <prefix>.s (fp32 [TM, TN]) and <prefix>.deq
// (fp32 [M, N]) for the caller to compare with the CPU oracle.
//
// usage: gpu_client <in.bf16> M N bm bn <prefix>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fp8bq.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    const hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

#define FP8BQ_OK_(call)                                                           \
  do {                                                                            \
    const int s_ = (call);                                                        \
    if (s_ != FP8BQ_OK) {                                                         \
      std::fprintf(stderr, "%s failed: %s (hip error %d)\n", #call,               \
                   fp8bq_status_string(s_), fp8bq_last_hip_error());              \
      return 3;                                                                   \
    }                                                                             \
  } while (0)

static bool write_file(const char* path, const void* p, size_t n) {
  FILE* f = std::fopen(path, "wb");
  if (f == nullptr) return false;
  const bool ok = std::fwrite(p, 1, n, f) == n;
  return std::fclose(f) == 0 && ok;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: %s <in.bf16> M N bm bn <prefix>\n", argv[0]);
    return 1;
  }
  const int64_t M = std::atoll(argv[2]), N = std::atoll(argv[3]);
  const int32_t bm = std::atoi(argv[4]), bn = std::atoi(argv[5]);
  if (M < 1 || N < 1 || bm < 1 || bn < 1) return 1;
  const size_t n = static_cast<size_t>(M) * static_cast<size_t>(N);
  const size_t ns = static_cast<size_t>((M + bm - 1) / bm) * static_cast<size_t>((N + bn - 1) / bn);

  std::vector<uint16_t> x(n);
  FILE* f = std::fopen(argv[1], "rb");
  if (f == nullptr || std::fread(x.data(), 2, n, f) != n) {
    std::fprintf(stderr, "cannot read %zu BF16 values from %s\n", n, argv[1]);
    return 1;
  }
  std::fclose(f);

  void *dx = nullptr, *dq = nullptr, *dq2 = nullptr;
  float *ds = nullptr, *ds2 = nullptr, *ddeq = nullptr;
  HIP_OK(hipMalloc(&dx, 2 * n));
  HIP_OK(hipMalloc(&dq, n));
  HIP_OK(hipMalloc(&dq2, n));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&ds), 4 * ns));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&ds2), 4 * ns));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&ddeq), 4 * n));
  float* ddeq2 = nullptr;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&ddeq2), 8 * n));
  HIP_OK(hipMemcpy(dx, x.data(), 2 * n, hipMemcpyHostToDevice));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  FP8BQ_OK_(fp8bq_quantize(dx, M, N, bm, bn, dq, ds, st));

  hipGraph_t graph;
  hipGraphExec_t exec;
  fp8bq_tensor entry = {dx, dq2, ds2, M, N};
  HIP_OK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
  const int cap_status = fp8bq_quantize_many(&entry, 1, bm, bn, nullptr, 0, st);
  HIP_OK(hipStreamEndCapture(st, &graph));
  FP8BQ_OK_(cap_status);
  HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  for (int rep = 0; rep < 2; ++rep) {
    HIP_OK(hipMemsetAsync(dq2, 0xA5, n, st));
    HIP_OK(hipMemsetAsync(ds2, 0xFF, 4 * ns, st));
    HIP_OK(hipGraphLaunch(exec, st));
  }

  FP8BQ_OK_(fp8bq_dequantize(dq, ds, M, N, bm, bn, ddeq, FP8BQ_OUT_F32, st));
  const fp8bq_dq_tensor dql[2] = {{dq, ds, ddeq2, M, N}, {dq2, ds2, ddeq2 + n, M, N}};
  FP8BQ_OK_(fp8bq_dequantize_many(dql, 2, bm, bn, FP8BQ_OUT_F32, st));
  HIP_OK(hipStreamSynchronize(st));

  std::vector<uint8_t> q(n), q2(n);
  std::vector<float> s(ns), s2(ns), deq(n);
  HIP_OK(hipMemcpy(q.data(), dq, n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(q2.data(), dq2, n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(s.data(), ds, 4 * ns, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(s2.data(), ds2, 4 * ns, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(deq.data(), ddeq, 4 * n, hipMemcpyDeviceToHost));
  std::vector<float> deq2(2 * n);
  HIP_OK(hipMemcpy(deq2.data(), ddeq2, 8 * n, hipMemcpyDeviceToHost));
  if (std::memcmp(deq.data(), deq2.data(), 4 * n) != 0 ||
      std::memcmp(deq.data(), deq2.data() + n, 4 * n) != 0) {
    std::fprintf(stderr, "grouped dequantization differs from the single call\n");
    return 5;
  }
  if (std::memcmp(q.data(), q2.data(), n) != 0 || std::memcmp(s.data(), s2.data(), 4 * ns) != 0) {
    std::fprintf(stderr, "graph replay differs from the direct call\n");
    return 4;
  }

  const std::string prefix = argv[6];
  if (!write_file((prefix + ".q").c_str(), q.data(), n) ||
      !write_file((prefix + ".s").c_str(), s.data(), 4 * ns) ||
      !write_file((prefix + ".deq").c_str(), deq.data(), 4 * n)) {
    std::fprintf(stderr, "cannot write outputs under %s\n", argv[6]);
    return 1;
  }
  HIP_OK(hipGraphExecDestroy(exec));
  HIP_OK(hipGraphDestroy(graph));
  HIP_OK(hipStreamDestroy(st));
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dq2));
  HIP_OK(hipFree(ds));
  HIP_OK(hipFree(ds2));
  HIP_OK(hipFree(ddeq));
  HIP_OK(hipFree(ddeq2));
  std::printf("gpu client ok: %lldx%lld at [%d,%d], graph replays equal\n",
              static_cast<long long>(M), static_cast<long long>(N), bm, bn);
  return 0;
}
