// A native client of libfp8bq on the GPU, with no Python and no torch.
// It reads a BF16 matrix from a file and, on a stream of its own:
//   1. quantizes it with fp8bq_quantize;
//   2. captures fp8bq_quantize_many (one entry, other outputs) in a HIP
//      graph and replays it twice, refilling those outputs with a pattern
//      before each replay (eagerly, outside the graph);
//   3. dequantizes the result of step 1 to fp32 with fp8bq_dequantize, and
//      both results again with one fp8bq_dequantize_many call;
//   4. quantizes the first tile row of the input as 520 and then 515 entries
//      of fp8bq_quantize_many_noalloc (more than 512: the library's own
//      device table), each into outputs of its own;
//   5. quantizes the input as two row shards cut at row M/2 + 1 (inside a
//      tile row unless that row is a multiple of bm): fp8bq_row_shards_begin
//      records an event after the edge rows' maxima, a second stream waits
//      for it and exchanges the shared tile row's maxima (through the host),
//      and fp8bq_row_shards_finish runs once that stream is done.
// It checks that the quantizations, and all three dequantizations, agree
// byte for byte (every entry of step 4 with the first tile row of step 1,
// the shards of step 5 with the rows and scale rows of step 1) and writes
// <prefix>.q (uint8 [M, N]), <prefix>.s (fp32 [TM, TN]) and <prefix>.deq
// (fp32 [M, N]) for the caller to compare with the CPU oracle.
//
// usage: gpu_client <in.bf16> M N bm bn <prefix>
#include <hip/hip_runtime.h>

#include <algorithm>
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

  // 4. the first tile row as many entries of the call that allocates nothing
  const int64_t R = M < bm ? M : bm;
  const size_t rn = static_cast<size_t>(R) * static_cast<size_t>(N);
  const size_t rs = static_cast<size_t>((N + bn - 1) / bn);
  const int kEntries = 520;
  void* dq3 = nullptr;
  float* ds3 = nullptr;
  HIP_OK(hipMalloc(&dq3, kEntries * rn));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&ds3), 4 * kEntries * rs));
  std::vector<fp8bq_tensor> list(kEntries);
  for (int i = 0; i < kEntries; ++i) {
    list[i] = {dx, static_cast<uint8_t*>(dq3) + i * rn, ds3 + i * rs, R, N};
  }
  std::vector<uint8_t> q3(kEntries * rn);
  std::vector<float> s3(kEntries * rs);
  for (const int count : {kEntries, kEntries - 5}) {
    HIP_OK(hipMemsetAsync(dq3, 0x5A, kEntries * rn, st));
    HIP_OK(hipMemsetAsync(ds3, 0xFF, 4 * kEntries * rs, st));
    FP8BQ_OK_(fp8bq_quantize_many_noalloc(list.data(), count, bm, bn, st));
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(q3.data(), dq3, kEntries * rn, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(s3.data(), ds3, 4 * kEntries * rs, hipMemcpyDeviceToHost));
    for (int i = 0; i < count; ++i) {
      if (std::memcmp(q3.data() + i * rn, q.data(), rn) != 0 ||
          std::memcmp(s3.data() + i * rs, s.data(), 4 * rs) != 0) {
        std::fprintf(stderr, "no-alloc entry %d of %d differs from the direct call\n", i, count);
        return 6;
      }
    }
  }
  HIP_OK(hipFree(dq3));
  HIP_OK(hipFree(ds3));

  // 5. two row shards, the exchange of their shared tile row on a second stream
  const int64_t cut = M / 2 + 1 < M ? M / 2 + 1 : M;
  const int64_t TN = (N + bn - 1) / bn;
  const int64_t r0s[2] = {0, cut};
  int64_t tml[2], tops[2], bots[2];
  fp8bq_row_shard rsh[2];
  void* dq5 = nullptr;
  float* ds5[2] = {nullptr, nullptr};
  HIP_OK(hipMalloc(&dq5, n));
  for (int k = 0; k < 2; ++k) {
    const int64_t rows = k == 0 ? cut : M - cut;
    const int32_t rp = static_cast<int32_t>(r0s[k] % bm);
    FP8BQ_OK_(fp8bq_row_shard_edges(rows, bm, rp, &tops[k], &bots[k]));
    tml[k] = rows == 0 ? 0 : (rp + rows + bm - 1) / bm;
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&ds5[k]), 4 * static_cast<size_t>(std::max<int64_t>(tml[k], 1) * TN)));
    rsh[k] = {static_cast<const uint16_t*>(dx) + r0s[k] * N, static_cast<uint8_t*>(dq5) + r0s[k] * N,
              ds5[k], tops[k] > 0 ? ds5[k] : nullptr, bots[k] > 0 ? ds5[k] + (tml[k] - 1) * TN : nullptr,
              rows, N, rp, 0};
  }
  hipStream_t side;
  hipEvent_t maxima, exchanged;
  HIP_OK(hipStreamCreate(&side));
  HIP_OK(hipEventCreateWithFlags(&maxima, hipEventDisableTiming));
  HIP_OK(hipEventCreateWithFlags(&exchanged, hipEventDisableTiming));
  HIP_OK(hipMemsetAsync(dq5, 0x5A, n, st));
  FP8BQ_OK_(fp8bq_row_shards_begin(rsh, 2, bm, bn, nullptr, 0, maxima, st));
  HIP_OK(hipStreamWaitEvent(side, maxima, 0));
  if (bots[0] > 0 && tops[1] > 0) {  // the first shard's last rows share a tile row with the second's first
    std::vector<float> a(TN), b(TN);
    HIP_OK(hipMemcpyAsync(a.data(), rsh[0].bottom_amax, 4 * TN, hipMemcpyDeviceToHost, side));
    HIP_OK(hipMemcpyAsync(b.data(), rsh[1].top_amax, 4 * TN, hipMemcpyDeviceToHost, side));
    HIP_OK(hipStreamSynchronize(side));
    for (int64_t j = 0; j < TN; ++j) a[j] = std::max(a[j], b[j]);
    HIP_OK(hipMemcpyAsync(rsh[0].bottom_amax, a.data(), 4 * TN, hipMemcpyHostToDevice, side));
    HIP_OK(hipMemcpyAsync(rsh[1].top_amax, a.data(), 4 * TN, hipMemcpyHostToDevice, side));
    HIP_OK(hipStreamSynchronize(side));
  }
  HIP_OK(hipEventRecord(exchanged, side));
  HIP_OK(hipStreamWaitEvent(st, exchanged, 0));
  FP8BQ_OK_(fp8bq_row_shards_finish(rsh, 2, bm, bn, st));
  HIP_OK(hipStreamSynchronize(st));
  std::vector<uint8_t> q5(n);
  HIP_OK(hipMemcpy(q5.data(), dq5, n, hipMemcpyDeviceToHost));
  if (std::memcmp(q5.data(), q.data(), n) != 0) {
    std::fprintf(stderr, "row shards cut at %lld differ from the direct call\n", static_cast<long long>(cut));
    return 7;
  }
  for (int k = 0; k < 2; ++k) {
    std::vector<float> s5(static_cast<size_t>(tml[k] * TN));
    HIP_OK(hipMemcpy(s5.data(), ds5[k], 4 * s5.size(), hipMemcpyDeviceToHost));
    if (std::memcmp(s5.data(), s.data() + (r0s[k] / bm) * TN, 4 * s5.size()) != 0) {
      std::fprintf(stderr, "row shard %d's scales differ from the direct call's\n", k);
      return 7;
    }
  }
  HIP_OK(hipEventDestroy(maxima));
  HIP_OK(hipEventDestroy(exchanged));
  HIP_OK(hipStreamDestroy(side));
  HIP_OK(hipFree(dq5));
  HIP_OK(hipFree(ds5[0]));
  HIP_OK(hipFree(ds5[1]));

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
  std::printf("gpu client ok: %lldx%lld at [%d,%d], graph replays, no-alloc entries and row shards equal\n",
              static_cast<long long>(M), static_cast<long long>(N), bm, bn);
  return 0;
}
