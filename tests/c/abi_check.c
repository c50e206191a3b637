/* A plain C client of libfp8bq: compiles against include/fp8bq.h in strict
 * C99 and exercises argument checking only (fake addresses that every call
 * must reject before touching a device).  Prints "abi ok" on success. */
#include <stdint.h>
#include <stdio.h>

#include "fp8bq.h"

#define X ((const void*)(uintptr_t)0x1000000000ull)
#define Q ((void*)(uintptr_t)0x2000000000ull)
#define S ((float*)(uintptr_t)0x3000000000ull)

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: got %d (%s), want %d\n", what, got, fp8bq_status_string(got), want);
    ++failures;
  }
}

int main(void) {
  fp8bq_tensor t[2];
  t[0].x = X; t[0].q = Q; t[0].scale_inv = S; t[0].M = 256; t[0].N = 256;
  t[1] = t[0];
  t[1].M = -1;
  expect(fp8bq_quantize(X, -1, 128, 128, 128, Q, S, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "negative M");
  expect(fp8bq_quantize(X, 128, 128, 0, 128, Q, S, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "bm < 1");
  expect(fp8bq_quantize(NULL, 128, 128, 128, 128, Q, S, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "null x");
  expect(fp8bq_quantize(X, 128, 128, 128, 128, (void*)X, S, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "q overlaps x");
  expect(fp8bq_quantize(NULL, 0, 128, 128, 128, NULL, NULL, NULL), FP8BQ_OK, "empty");
  expect(fp8bq_quantize_many(t, 2, 128, 128, NULL, 0, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "bad entry");
  expect(fp8bq_quantize_many(t, -1, 128, 128, NULL, 0, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "count < 0");
  expect((int)fp8bq_many_workspace_bytes(FP8BQ_MANY_ARGS_MAX), 0, "no workspace up to the arg limit");
  if (fp8bq_many_workspace_bytes(FP8BQ_MANY_ARGS_MAX + 1) == 0) {
    printf("FAIL workspace size for a large group\n");
    ++failures;
  }
  expect(fp8bq_dequantize(Q, S, 128, 128, 128, 128, Q, FP8BQ_OUT_F32, NULL),
         FP8BQ_ERR_INVALID_ARGUMENT, "dequant out overlaps q");
  expect(fp8bq_tile_amax(X, 128, 128, 128, 128, 128, 0, S, NULL), FP8BQ_ERR_INVALID_ARGUMENT,
         "phase out of range");
  expect(fp8bq_quantize_amax(X, 128, 128, 128, 128, 0, 0, NULL, Q, S, NULL),
         FP8BQ_ERR_INVALID_ARGUMENT, "null amax");
  {
    fp8bq_shard sh[2];
    sh[0].x = X; sh[0].q = Q; sh[0].amax = S; sh[0].scale_inv = S;
    sh[0].M = 256; sh[0].N = 256; sh[0].row_phase = 64; sh[0].col_phase = 0;
    sh[1] = sh[0];
    sh[1].row_phase = 128;
    expect(fp8bq_tile_amax_many(sh, 2, 128, 128, NULL), FP8BQ_ERR_INVALID_ARGUMENT,
           "shard phase out of range");
    expect(fp8bq_quantize_amax_many(NULL, 1, 128, 128, NULL), FP8BQ_ERR_INVALID_ARGUMENT,
           "null shard list");
    expect(fp8bq_quantize_amax_many(sh, 0, 128, 128, NULL), FP8BQ_OK, "no shards");
  }
  expect(fp8bq_encode_e4m3(NULL, Q, 4, NULL), FP8BQ_ERR_INVALID_ARGUMENT, "null y");
  {
    fp8bq_dq_tensor dq[2] = {{Q, S, (void*)(uintptr_t)0x1000000000ull, 128, 128},
                             {Q, S, (void*)(uintptr_t)0x1000000002ull, 128, 128}};
    expect(fp8bq_dequantize_many(dq, 2, 128, 128, FP8BQ_OUT_F32, NULL), FP8BQ_ERR_INVALID_ARGUMENT,
           "grouped dequant, misaligned out");
    expect(fp8bq_dequantize_many(dq, 0, 128, 128, FP8BQ_OUT_F32, NULL), FP8BQ_OK, "no dequant entries");
  }
  expect(fp8bq_set_resident_wait_us(-1), FP8BQ_ERR_INVALID_ARGUMENT, "negative wait");
  expect(fp8bq_set_resident_wait_us(2000), FP8BQ_OK, "default wait");
  expect(fp8bq_last_hip_error(), 0, "no HIP call made");
  if (failures == 0) printf("abi ok\n");
  return failures == 0 ? 0 : 1;
}
