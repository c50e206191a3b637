/*
 * fp8bq — blockwise FP8 (OCP e4m3fn) weight quantization for AMD MI355X (gfx950).
 *
 * The operation is the blockwise cast on the documentation page
 * "fp8_kernel.py — FP8 量化内核" (verl/utils/kernel/fp8_kernel.py):
 *   - section 1, unified entry point: [M, N] high-precision data and a
 *     [BLOCK_M, BLOCK_N] block size in, FP8 data and a descale per block out;
 *   - section 2, Triton implementation: per block, amax = max(max|x|, eps),
 *     s = amax / 448, q = clamp(x * (1/s), -448, 448) cast to float8_e4m3fn,
 *     s stored as the descale.
 * The grouped call serves the streaming loop of the page "vllm_fp8_utils.py"
 * (section 3, quant_weights), which quantizes a list of weights with one
 * block size and pairs each weight with a "<name>_scale_inv" tensor.
 *
 * Arithmetic (bit-exact, deterministic):
 *   a = max(amax, FP8BQ_EPS)      amax over the tile's valid elements (exact)
 *   s = a / 448                   correctly rounded binary32 division
 *   r = 1 / s                     correctly rounded binary32 division
 *   y = x * r                     binary32, round to nearest even
 *   q = e4m3fn(clamp(y, -448, 448))   round to nearest even, sign kept
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronizes on these calls; work is
 *     enqueued on `stream` (a hipStream_t; NULL means the null stream) and
 *     results are ready when that stream reaches the call.
 *   - x is BF16, contiguous row-major [M, N] (row pitch N elements).
 *   - q is one byte per element, contiguous row-major [M, N]; every byte is
 *     written.  Bytes are OCP e4m3fn codes (torch.float8_e4m3fn); 0x7F and
 *     0xFF (NaN) are never produced for finite input.
 *   - scale_inv is fp32, contiguous row-major [ceil(M/bm), ceil(N/bn)];
 *     every entry is written.  Dequantization is decode(q) * scale_inv.
 *   - Outputs must not overlap each other or x (checked per tensor).
 *   - Non-finite input (NaN, Inf) is outside the contract; the output for
 *     such a tile is unspecified but every write stays inside q/scale_inv.
 *   - M == 0 or N == 0 (or count == 0) returns FP8BQ_OK without touching
 *     the device.
 *   - All argument checks run before any HIP call.  The first compute call
 *     on a device checks that it is a gfx950 (the capability check the
 *     relations section of the fp8_kernel.py page delegates to device.py).
 *   - Any block size bm, bn >= 1 and any alignment are accepted.  Blocks
 *     [128,128], [64,64] and [1,128] with N % 8 == 0, a 16-byte aligned x
 *     and an 8-byte aligned q take the vectorized kernels; tiles of more
 *     than 65536 elements take two passes (maxima, then quantization), and
 *     between the passes q holds partial maxima until the codes replace
 *     them; all other cases take a general one-workgroup-per-tile kernel.
 *     A whole tensor with one tile (bm >= M, bn >= N) of at least 2^20
 *     values, aligned as above, that fits in the registers of the grid the
 *     device holds at once (about 50 M values on an MI355X) is read once
 *     and held in registers while the workgroups agree on its maximum
 *     (fp8bq_set_resident_wait_us); during the call q's bytes 0..7 and
 *     128..135 and scale_inv hold that handshake until the results replace
 *     them.  Results are identical whichever kernel runs.
 *   - Thread safety: calls may be made from several host threads; each
 *     thread has its own fp8bq_last_hip_error().
 */
#ifndef FP8BQ_H
#define FP8BQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BQ_E4M3_MAX 448.0f
/* Floor of the tile maximum.  The page names eps without a value; 1e-10 is
 * the value this library uses (an all-zero tile gets scale fl32(eps/448)). */
#define FP8BQ_EPS 1e-10f

enum fp8bq_status {
  FP8BQ_OK = 0,
  FP8BQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bm/bn < 1, overlap, size overflow */
  FP8BQ_ERR_UNSUPPORTED_DEVICE = 2, /* the current device is not a gfx950 */
  FP8BQ_ERR_WORKSPACE = 3,        /* workspace null, too small or not 16-byte aligned */
  FP8BQ_ERR_HIP = 4               /* a HIP call failed; see fp8bq_last_hip_error() */
};

/*
 * Quantize one BF16 matrix.
 *   x          device, BF16 [M, N] row-major
 *   M, N       rows and columns (>= 0, each < 2^31)
 *   bm, bn     block rows and columns (>= 1); [128,128] is the weight
 *              default, [1,128] the per-row-group (activation-style) shape
 *   q          device, uint8 [M, N] row-major (e4m3fn codes)
 *   scale_inv  device, fp32 [ceil(M/bm), ceil(N/bn)] row-major
 *   stream     hipStream_t to enqueue on (NULL = null stream)
 * Returns an fp8bq_status.
 */
int fp8bq_quantize(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn,
                   void* q, float* scale_inv, void* stream);

/* One entry of a grouped call (fields as in fp8bq_quantize). */
typedef struct fp8bq_tensor {
  const void* x;
  void* q;
  float* scale_inv;
  int64_t M;
  int64_t N;
} fp8bq_tensor;

/* Maximum number of tensors whose descriptor table fp8bq_quantize_many passes
 * in the kernel arguments (no workspace, no host-to-device copy). */
#define FP8BQ_MANY_ARGS_MAX 512

/* Device workspace bytes fp8bq_quantize_many needs for `count` tensors: 0 for
 * count <= FP8BQ_MANY_ARGS_MAX (the table rides in the kernel arguments). */
size_t fp8bq_many_workspace_bytes(int32_t count);

/*
 * Quantize a list of BF16 matrices that share one block size, in one kernel
 * launch (the grouped form of the per-weight loop); entries with tiles of
 * more than 65536 elements add three launches per 128 such entries.
 *   list             HOST array of `count` entries; its contents are captured
 *                    before the call returns (into the kernel arguments, or
 *                    copied into `workspace` on `stream`), so the caller may
 *                    reuse or free it afterwards.  While `stream` is
 *                    capturing a graph, a call of more than
 *                    FP8BQ_MANY_ARGS_MAX entries enqueues no copy: it
 *                    launches once per run of at most that many entries,
 *                    each with its table in the kernel arguments (the
 *                    workspace is then left untouched)
 *   count            number of entries (>= 0)
 *   bm, bn           block size shared by every entry
 *   workspace        device buffer of at least
 *                    fp8bq_many_workspace_bytes(count) bytes, 16-byte
 *                    aligned, untouched until the launch on `stream` has
 *                    finished; may be NULL when that size is 0 (count <=
 *                    FP8BQ_MANY_ARGS_MAX)
 *   workspace_bytes  its size
 *   stream           hipStream_t (NULL = null stream)
 * Entries with M == 0 or N == 0 are skipped.  Entries whose tiles exceed
 * 65536 elements are quantized by the two-pass kernels (grouped, up to 128
 * entries per launch, before the grouped launch of the others).  Outputs of
 * different entries must not overlap each other or any entry's x (not
 * checked across entries).
 * Returns an fp8bq_status; on an argument error nothing is enqueued.
 */
int fp8bq_quantize_many(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Largest list fp8bq_quantize_many_noalloc takes. */
#define FP8BQ_NOALLOC_MAX_TENSORS 16384

/*
 * fp8bq_quantize_many without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and rules as
 * fp8bq_quantize_many, whose kernels it launches; where that call copies the
 * descriptor table of more than FP8BQ_MANY_ARGS_MAX tensors into the
 * caller's workspace, this one copies it into device memory the library
 * holds: one block of 1,179,904 bytes per GPU it runs on, kept until the
 * process ends.  It calls no hipMalloc, hipFree or other allocating routine.
 *   count  0 .. FP8BQ_NOALLOC_MAX_TENSORS; larger lists return
 *          FP8BQ_ERR_WORKSPACE with nothing enqueued
 * Every call on one GPU shares that block, and a call's copy and launch read
 * it until the launch ends: calls that overlap on one GPU (other streams,
 * other threads, without ordering between them) race.  Order them on one
 * stream, or use fp8bq_quantize_many with a workspace per stream.  Lists of
 * at most FP8BQ_MANY_ARGS_MAX tensors, and any list while `stream` is
 * capturing a graph, carry their table in the kernel arguments and do not
 * touch the block.  Nothing in it needs to start at zero: each call writes
 * the whole table it reads.
 * Returns an fp8bq_status; on an argument error nothing is enqueued.
 */
int fp8bq_quantize_many_noalloc(const fp8bq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                                void* stream);

/*
 * Shards and large tiles.  A shard is an [M, N] sub-matrix of a larger
 * matrix whose element (0,0) sits at (row_phase, col_phase) inside a tile of
 * the full matrix's [bm, bn] grid (0 <= row_phase < bm, 0 <= col_phase < bn;
 * both 0 for a whole matrix or a tile-aligned shard).  Its local tile grid is
 * TMl = ceil((row_phase + M) / bm) by TNl = ceil((col_phase + N) / bn).
 *
 * fp8bq_tile_amax writes amax[TMl, TNl] (fp32, device): the largest |x| over
 * the part of each tile inside this shard -- the first step of the blockwise
 * cast of the fp8_kernel.py page (section 2) restricted to one shard.  Tiles
 * shared by several shards (rows or columns cut inside a tile) get their
 * full maximum as the max over those shards' partial maxima; the values are
 * exact BF16 magnitudes, so the combination is exact in any order.
 *
 * fp8bq_quantize_amax quantizes the shard with the given whole-tile maxima
 * and writes q [M, N] and scale_inv [TMl, TNl] (the shard's rows of the full
 * scale grid).  `amax` may be the same array as `scale_inv` (converted in
 * place), but must not partly overlap it.  Given the full maxima, every
 * shard's bytes equal the corresponding bytes of quantizing the whole matrix.
 *
 * The same two passes serve fp8bq_quantize / fp8bq_quantize_many for tiles
 * of more than 65536 elements (e.g. one scale per tensor: bm = M, bn = N);
 * there the partial maxima of pass 1 go to slots in q (one per workgroup,
 * no atomics), a small kernel reduces them to the scales, and pass 2
 * overwrites q with the codes.
 * Both calls enqueue on `stream`; the pointers follow the conventions above.
 */
int fp8bq_tile_amax(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn, int32_t row_phase,
                    int32_t col_phase, float* amax, void* stream);
int fp8bq_quantize_amax(const void* x, int64_t M, int64_t N, int32_t bm, int32_t bn,
                        int32_t row_phase, int32_t col_phase, const float* amax, void* q,
                        float* scale_inv, void* stream);

/* One shard of a grouped shard call (fields as in fp8bq_tile_amax and
 * fp8bq_quantize_amax; TMl x TNl is the shard's local tile grid). */
typedef struct fp8bq_shard {
  const void* x;     /* BF16 [M, N] row-major */
  void* q;           /* e4m3fn [M, N]; written by fp8bq_quantize_amax_many only */
  float* amax;       /* fp32 [TMl, TNl]: written by fp8bq_tile_amax_many, read by
                        fp8bq_quantize_amax_many */
  float* scale_inv;  /* fp32 [TMl, TNl]; written by fp8bq_quantize_amax_many only,
                        may be the same array as amax */
  int64_t M;
  int64_t N;
  int32_t row_phase;
  int32_t col_phase;
} fp8bq_shard;

/*
 * Grouped forms of fp8bq_tile_amax and fp8bq_quantize_amax over a list of
 * shards that share one block size: the same results as one call per entry,
 * in fewer launches.  For the quantize-before-gather of sharded weights
 * (every rank quantizes its own slabs; only tiles cut by a slab boundary
 * need their partial maxima exchanged), which the sharding discussion of
 * the page "Using FP8 inference in long response vllm rollouts" points to.
 *   list    HOST array of `count` entries, read before the call returns
 *   count   number of entries (>= 0); entries with M == 0 or N == 0 are skipped
 *   bm, bn  block size shared by every entry
 *   stream  hipStream_t (NULL = null stream)
 * Every entry is checked as the single call checks it before anything is
 * enqueued.  Entries whose tiles hold at most 16,384 elements, with tile
 * columns on 8-element boundaries (x 16-byte and q 8-byte aligned; N, bn and
 * col_phase multiples of 8), share launches of up to 512 entries with the
 * table in the kernel arguments (graph-capturable, no workspace); other
 * entries take their own two-pass launches.  Outputs of different entries
 * must not overlap each other or any entry's x (not checked across entries).
 * Returns an fp8bq_status.
 */
int fp8bq_tile_amax_many(const fp8bq_shard* list, int32_t count, int32_t bm, int32_t bn,
                         void* stream);
int fp8bq_quantize_amax_many(const fp8bq_shard* list, int32_t count, int32_t bm, int32_t bn,
                             void* stream);

/*
 * Row shards, with the exchange confined to the tile rows that shards share.
 * A row shard holds whole rows of a matrix (the full width N, column phase
 * 0), its first row at row_phase inside a tile row: the weights split
 * across ranks by rows before the gather (the sharding discussion of the
 * page "Using FP8 inference in long response vllm rollouts").  Only its
 * first `top` and last `bottom` rows (fp8bq_row_shard_edges) lie in tile
 * rows that other shards may hold too; the tile rows between them are whole
 * and need no exchange.  The quantize-before-gather of such shards runs as
 *   1. fp8bq_row_shards_begin: the partial maxima of each shard's edge rows
 *      (top_amax, bottom_amax; the tile maxima of fp8bq_tile_amax), then
 *      the whole tile rows between them quantized in one pass (their q rows
 *      and scale rows, as fp8bq_quantize_many);
 *   2. the caller's exchange: each edge's maxima replaced, element by
 *      element, by the max over every shard that holds part of that tile
 *      row (left as they are where no other shard does).  It may run on
 *      another stream once `maxima_event` has completed, beside the
 *      whole-tile-row work of step 1;
 *   3. fp8bq_row_shards_finish: the edge rows quantized with those maxima
 *      (their q rows and the first / last scale row, as
 *      fp8bq_quantize_amax), on a stream ordered after the exchange.
 * Every byte and scale then equals quantizing the whole matrix.  Whole tile
 * rows are read once and edge rows twice, where fp8bq_tile_amax_many and
 * fp8bq_quantize_amax_many read every row twice.
 */
typedef struct fp8bq_row_shard {
  const void* x;       /* BF16 [M, N] row-major */
  void* q;             /* e4m3fn [M, N] */
  float* scale_inv;    /* fp32 [TMl, TN]: TMl = ceil((row_phase + M) / bm), TN = ceil(N / bn) */
  float* top_amax;     /* fp32 [TN], the tile row of the first `top` rows (unused when
                          top == 0); may be scale_inv's first row, converted in place */
  float* bottom_amax;  /* fp32 [TN], the tile row of the last `bottom` rows (unused when
                          bottom == 0); may be scale_inv's last row */
  int64_t M;
  int64_t N;
  int32_t row_phase;   /* 0 <= row_phase < bm */
  int32_t reserved;    /* ignored */
} fp8bq_row_shard;

/* The edge rows of a row shard of M rows at row_phase:
 * *top = min(M, (bm - row_phase) % bm) rows at its start and
 * *bottom = (M - *top) % bm rows at its end.  Host arithmetic only; returns
 * FP8BQ_ERR_INVALID_ARGUMENT unless 0 <= M <= INT32_MAX, bm >= 1 and
 * 0 <= row_phase < bm. */
int fp8bq_row_shard_edges(int64_t M, int32_t bm, int32_t row_phase, int64_t* top, int64_t* bottom);

/*
 *   list          HOST array of `count` entries, read before the call returns
 *   count         number of entries (>= 0); entries with M == 0 or N == 0 are skipped
 *   bm, bn        block size shared by every entry
 *   workspace     device memory for the table of the shards' whole-tile parts, as
 *   workspace_bytes  in fp8bq_quantize_many: fp8bq_many_workspace_bytes(count)
 *                 bytes are always enough (NULL / 0 for count <= FP8BQ_MANY_ARGS_MAX)
 *   maxima_event  hipEvent_t recorded on `stream` after the edge maxima, before the
 *                 whole-tile-row launches (NULL: none)
 *   stream        hipStream_t (NULL = null stream)
 * Every entry is checked before anything is enqueued: ranges, null pointers,
 * alignment (x 2-byte, scale_inv and the maxima 4-byte), and the overlaps of
 * x, q, scale_inv, top_amax and bottom_amax within the entry (not across
 * entries).  Returns an fp8bq_status.
 */
int fp8bq_row_shards_begin(const fp8bq_row_shard* list, int32_t count, int32_t bm, int32_t bn,
                           void* workspace, size_t workspace_bytes, void* maxima_event,
                           void* stream);
int fp8bq_row_shards_finish(const fp8bq_row_shard* list, int32_t count, int32_t bm, int32_t bn,
                            void* stream);

/* Output element type of fp8bq_dequantize. */
enum fp8bq_out_dtype {
  FP8BQ_OUT_F32 = 0,  /* float32 */
  FP8BQ_OUT_BF16 = 1  /* bfloat16, rounded to nearest (ties to even) from the fp32 product */
};

/*
 * Dequantize: out[i,j] = decode(q[i,j]) * scale_inv[i/bm, j/bn], the
 * consumer side of the descale (the "descale" output of the fp8_kernel.py
 * page, section 1; the "<name>_scale_inv" tensor of the vllm_fp8_utils.py
 * page, section 3).  The product is rounded once to fp32; FP8BQ_OUT_BF16
 * rounds that fp32 value to BF16 (nearest, ties to even).
 *   q          device, e4m3fn bytes [M, N] row-major
 *   scale_inv  device, fp32 [ceil(M/bm), ceil(N/bn)] row-major
 *   out        device, [M, N] row-major of out_dtype (fp32 or BF16), aligned
 *              to its element size; must not overlap q or scale_inv
 * Any shape, block size and alignment; with G = 4 (fp32) or 8 (BF16),
 * N % G == 0, bn % G == 0, q aligned to G bytes and out to 16 bytes take the
 * vectorized kernel.  NaN codes decode to NaN.
 */
int fp8bq_dequantize(const void* q, const float* scale_inv, int64_t M, int64_t N, int32_t bm,
                     int32_t bn, void* out, int32_t out_dtype, void* stream);

/* One tensor of a grouped dequantization (40 bytes, no padding). */
typedef struct {
  const void* q;          /* device, e4m3fn bytes [M, N] row-major */
  const float* scale_inv; /* device, fp32 [ceil(M/bm), ceil(N/bn)] row-major */
  void* out;              /* device, [M, N] row-major of the call's out_dtype */
  int64_t M;
  int64_t N;
} fp8bq_dq_tensor;

/*
 * fp8bq_dequantize over a list of tensors that share one block size and one
 * output type: the same results as one call per entry, in fewer launches
 * (the consumer side of a grouped fp8bq_quantize_many, e.g. the round trip
 * of a whole layer list).
 *   list       HOST array of `count` entries, read before the call returns
 *   count      number of entries (>= 0); entries with M == 0 or N == 0 are skipped
 *   bm, bn     block size shared by every entry
 *   out_dtype  FP8BQ_OUT_F32 or FP8BQ_OUT_BF16, for every entry
 * Every entry is checked as the single call checks it before anything is
 * enqueued.  Entries that take the vector kernel share launches of up to 256
 * entries with the table in the kernel arguments (no workspace,
 * graph-capturable); the others take their own element-wise launches.
 * Outputs of different entries must not overlap each other or any entry's
 * inputs (not checked across entries).  Returns an fp8bq_status.
 */
int fp8bq_dequantize_many(const fp8bq_dq_tensor* list, int32_t count, int32_t bm, int32_t bn,
                          int32_t out_dtype, void* stream);

/*
 * The final cast alone (clamp to +-448, round to e4m3fn), for checking the
 * hardware convert over every float32 input.
 *   y  device, fp32 [n];  q  device, uint8 [n];  n >= 0.
 */
int fp8bq_encode_e4m3(const float* y, void* q, int64_t n, void* stream);

/*
 * Longest time a workgroup of the one-scale-per-tensor kernel held in
 * registers waits for the tensor-wide maximum (the page "fp8_kernel.py — FP8
 * 量化内核", section 2: the block maximum, here over one block that spans the
 * tensor) before it reads all of x and computes that maximum itself.  The
 * wait only runs long when the launch's workgroups are not all resident at
 * once (e.g. beside another kernel); the results are the same either way.
 *   microseconds  0 .. 2^40; default 2000.  0 makes every workgroup but the
 *                 last to arrive compute the maximum itself (slow; for tests).
 * Process-wide; applies to launches enqueued after the call.  Returns
 * FP8BQ_OK or FP8BQ_ERR_INVALID_ARGUMENT; touches no device.
 */
int fp8bq_set_resident_wait_us(int64_t microseconds);

/* Static English text for a status code (never NULL). */
const char* fp8bq_status_string(int status);

/* hipError_t of the last failed HIP call made by this thread inside the
 * library (0 if none). */
int fp8bq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_H */
