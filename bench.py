"""Benchmark: blockwise FP8 quantization throughput on one MI355X.

A step is one pass of the whole path over one batch of synthetic weights:
by default the 36-layer Qwen3-8B-shaped dense weight set (252 BF16 tensors,
6.95e9 values, 13.9 GB), quantized at block [128,128] in ONE grouped launch
(``fp8bq_quantize_many``), inputs already resident in HBM.

Reported value: algorithmic GB/s = (2 B read + 1 B written per element +
4 B per tile scale) / step time.  The JSON line also carries:
  roofline      the grouped kernel's achieved bytes per launch / its mean
                launch time (HIP events on the launch stream) vs 8 TB/s;
                `traffic` is the HBM byte count (FETCH_SIZE + WRITE_SIZE,
                scaled by a copy-kernel calibration) from the committed
                counter profile, or null if that profile is for other code;
  cpu_baseline  the CPU oracle timed on this host's cores (a pool of one
                worker process per available core, at most 16) over the
                whole benchmarked workload (or the first --cpu-values
                values), from BF16 bits in host memory to codes and scales;
  configs       (default run) the other weight sets in their own launch
                configurations, measured in the same run: the 256x256
                matrix, one dense layer (rotated copies, so the 256 MB
                Infinity Cache cannot serve it), the MoE set (one launch per
                layer) and the ragged set at each block size; wall and
                kernel time per step, GB/s and percent of the HBM peak;
  lib_sha       the fingerprint of the sources the loaded library was built from.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3]
                       [--workload dense|dense-layer|moe|ragged|vocab] [--block bm,bn]
                       [--copies N] [--per-tensor] [--no-cpu-baseline] [--cpu-values N]
                       [--no-configs] [--calibrate-copy] [--input-sha]

The first CPU-sample inputs are hashed (SHA-256 per tensor on stderr, and a
digest of those in cpu_baseline.sample_sha256); --input-sha hashes every
input of the workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from fp8_blockwise_weight_amd import build as _build  # noqa: E402  (stdlib only, no torch)

HBM_PEAK_GBS = 8000.0
METRIC = "blockwise FP8 quantize GB/s (bf16 in + fp8/scale out), % of HBM peak, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quantize_t128_dense36_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(M, N, bm, bn):
    TM, TN = -(-M // bm), -(-N // bn)
    return 3 * M * N + 4 * TM * TN


_code_only = _build.code_only
kernel_sha = _build.kernel_sha


def committed_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = None
    with open(TRAFFIC_FILE, encoding="utf-8") as f:
        for line in f:
            if line.startswith("TRAFFIC_JSON "):
                rec = json.loads(line[len("TRAFFIC_JSON "):])
    if not rec or rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def group_kernel_name(kind, count, flat=False):
    """Kernel a grouped call of `count` tensors launches (table in the kernel
    arguments up to 512 tensors, else in a workspace); `flat`: [1,128]
    tensors whose widths are all multiples of 128."""
    if count <= 512:
        cap = 8 if count <= 8 else (64 if count <= 64 else 512)
        if flat:
            return f"fp8bq::quantize_group_args_flat<{cap}>"
        return f"fp8bq::quantize_group_args<{kind},{cap}>"
    return f"fp8bq::quantize_group<{kind}>"


RESIDENT_MIN_VALUES = 1 << 20          # smallest tensor held in registers
RESIDENT_CAPACITY = 512 * 256 * 48 * 8  # values the MI355X holds in registers (2 workgroups per CU)


def call_kernels(specs, bm, bn, kind, flat):
    """(label, kernel launches) of one fp8bq_quantize_many call over `specs`,
    mirroring the library's choice (the label only; timing does not use it).
    Lists of whole one-tile tensors that fit in registers take a preparation
    launch and a persistent resident launch per 256 tensors; other tiles
    above 65536 elements take the grouped two-pass kernels, 3 launches per
    128 tensors."""
    n = len(specs)
    one_tile = all(sp.M <= bm and sp.N <= bn for sp in specs)
    big = all(min(sp.M, bm) * min(sp.N, bn) > 65536 for sp in specs)
    if one_tile and all(sp.N % 8 == 0 and RESIDENT_MIN_VALUES <= sp.M * sp.N <= RESIDENT_CAPACITY
                        for sp in specs):
        calls = -(-n // 256)
        if n == 1:
            return "fp8bq::resident_prep<256> + fp8bq::resident_quant<L>", 2
        return "fp8bq::resident_prep<256> + fp8bq::resident_group<256>", 2 * calls
    if big:
        return "fp8bq::big_group_max/reduce/quant<128>", 3 * -(-n // 128)
    return group_kernel_name(kind, n, flat), 1


def build_workload(name, dev, block=None):
    import torch  # noqa: F401
    from fp8_blockwise_weight_amd import workloads as wl

    if name == "dense":
        groups = [wl.c3()]
        desc = "qwen3-8b-shaped dense stack, 36 layers x 7 linears (252 tensors)"
    elif name == "dense-layer":
        groups = [wl.c2()]
        desc = "one qwen3-8b-shaped decoder layer (7 tensors)"
    elif name == "moe":
        groups = [wl.c4_layer(layer) for layer in range(wl.MOE_LAYERS)]
        desc = "moe 48 layers x 128 experts (w13 1536x2048, down 2048x768), one launch per layer"
    elif name == "ragged":
        groups = [[sp] for sp in wl.c5()]
        block = block or (128, 128)
        desc = (f"ragged 1000x3000, 4097x11008, 151937x4096, 77x128 at block "
                f"[{block[0]},{block[1]}], one launch each")
    elif name == "vocab":
        groups = [[sp] for sp in wl.c5() if sp.M == 151937]
        block = block or (128, 128)
        desc = f"151937x4096 (vocab-shaped) at block [{block[0]},{block[1]}]"
    else:
        raise SystemExit(f"unknown workload {name}")
    block = block or (128, 128)
    if block != (128, 128) and name in ("dense", "dense-layer", "moe"):
        desc += f" at block [{block[0]},{block[1]}]"
    return groups, block, desc


class Prepared:
    """A workload resident in HBM: its inputs (materialized once, cloned into
    ``copies`` sets whose steps rotate, so that a set smaller than the 256 MB
    Infinity Cache is not served from it), outputs and the host descriptor
    table of every grouped call."""

    def __init__(self, lib, groups, bm, bn, dev, sptr, copies=1):
        import torch

        import fp8_blockwise_weight_amd as fq
        from fp8_blockwise_weight_amd import workloads as wl

        t0 = time.perf_counter()
        self.lib, self.bm, self.bn, self.sptr = lib, bm, bn, sptr
        self.copies = max(1, int(copies))
        self.calls = []          # per copy: [(entries, count, workspace)] per grouped call
        self.keep = []           # copy 0: (xs, outs) per group
        hold = []
        base = [[wl.materialize(sp, dev) for sp in specs] for specs in groups]
        for c in range(self.copies):
            calls = []
            for xs0 in base:
                xs = xs0 if c == 0 else [x.clone() for x in xs0]
                outs = [(torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev),
                         torch.empty(fq.scale_shape(*x.shape, bm, bn), dtype=torch.float32, device=dev))
                        for x in xs]
                ws = torch.empty(max(fq.workspace_bytes(len(xs)), 1), dtype=torch.uint8, device=dev)
                calls.append((fq.make_entries(xs, outs), len(xs), ws))
                (self.keep if c == 0 else hold).append((xs, outs))
            self.calls.append(calls)
        self._hold = hold
        specs = [sp for g in groups for sp in g]
        self.bytes_per_step = sum(algorithmic_bytes(sp.M, sp.N, bm, bn) for sp in specs)
        self.elements = sum(sp.M * sp.N for sp in specs)
        self.tensors = len(specs)
        self.launches = len(groups)
        torch.cuda.synchronize()
        log(f"generated {self.tensors} tensors, {self.elements / 1e9:.3f} G values"
            f"{f' ({self.copies} copies)' if self.copies > 1 else ''} in {time.perf_counter() - t0:.1f}s")

    def step(self, i):
        lib, bm, bn, sptr = self.lib, self.bm, self.bn, self.sptr
        for arr, count, ws in self.calls[i % self.copies]:
            st = lib.fp8bq_quantize_many(arr, count, bm, bn, ws.data_ptr(), ws.numel(), sptr)
            if st != 0:
                raise RuntimeError(f"fp8bq_quantize_many failed: status {st}, "
                                   f"hip error {lib.fp8bq_last_hip_error()}")

    def time(self, steps, warmup, stream):
        """W untimed steps, then K steps timed by the wall clock between two
        device synchronizations, with HIP events on the launch stream around
        each step.  Returns (wall ms per step, [event ms per step])."""
        import torch

        for i in range(warmup):
            self.step(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            self.step(warmup + i)
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return wall * 1e3 / steps, [a.elapsed_time(b) for a, b in evs]


def config_records(lib, dev, sptr, stream, steps, warmup):
    """Throughput of the other weight sets, each measured here in its own
    launch configuration: the 256x256 matrix (launch-bound), one dense layer
    (three rotated copies: 1.7 GB between reuses of a buffer, well above the
    256 MB Infinity Cache), the MoE set (one grouped launch per layer) and the
    ragged set at each block size (one launch per matrix).  Wall time per step
    and kernel time per step (HIP events around the step) with their GB/s
    and percent of the HBM peak."""
    import torch
    from fp8_blockwise_weight_amd import workloads as wl

    plan = [
        ("c1_256x256", "C1 256x256 with planted outliers and a zero tile, [128,128] (launch-bound)",
         [wl.c1()], (128, 128), 1),
        ("c2_dense_layer", "C2 one qwen3-8b-shaped layer (7 tensors), [128,128], 3 rotated copies",
         [wl.c2()], (128, 128), 3),
        ("c4_moe", "C4 moe 48 layers x 128 experts (w13 1536x2048, down 2048x768), [128,128], "
                   "one grouped launch per layer", [wl.c4_layer(i) for i in range(wl.MOE_LAYERS)],
         (128, 128), 1),
    ]
    for blk in wl.RAGGED_BLOCKS:
        plan.append((f"c5_ragged_{blk[0]}x{blk[1]}",
                     f"C5 ragged 1000x3000, 4097x11008, 151937x4096, 77x128 at [{blk[0]},{blk[1]}], "
                     "one launch per matrix", [[sp] for sp in wl.c5()], blk, 1))
    out = {}
    for key, desc, groups, (bm, bn), copies in plan:
        prep = Prepared(lib, groups, bm, bn, dev, sptr, copies=copies)
        wall_ms, ev_ms = prep.time(steps, warmup, stream)
        gpu_ms = sum(ev_ms) / len(ev_ms)
        nbytes = prep.bytes_per_step
        rec = {
            "workload": desc,
            "block": [bm, bn],
            "tensors": prep.tensors,
            "launches_per_step": prep.launches,
            "rotated_copies": copies,
            "algorithmic_bytes_per_step": nbytes,
            "ms_per_step": round(wall_ms, 4),
            "GBps": round(nbytes / (wall_ms * 1e-3) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * nbytes / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "gpu_ms_per_step": round(gpu_ms, 4),
            "gpu_GBps": round(nbytes / (gpu_ms * 1e-3) / 1e9, 1),
            "gpu_pct_of_hbm_peak": round(100 * nbytes / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        }
        log(f"{key}: wall {wall_ms:.4f} ms/step ({rec['pct_of_hbm_peak']}% of peak), "
            f"events {gpu_ms:.4f} ms/step ({rec['gpu_pct_of_hbm_peak']}%)")
        out[key] = rec
        del prep
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense")
    ap.add_argument("--block", default=None, help="bm,bn for the ragged/vocab workloads")
    ap.add_argument("--op", default="quantize",
                    choices=["quantize", "dequant-f32", "dequant-bf16", "stream", "shard",
                             "shard-rows"],
                    help="quantize (default); time fp8bq_dequantize on the quantized workload; "
                         "time the streaming quant_weights loop over the workload in model "
                         "order with norm weights passed through; treat every tensor as a "
                         "shard at --phase and time fp8bq_tile_amax_many + "
                         "fp8bq_quantize_amax_many per group; or treat every tensor as a row "
                         "shard at the --phase row phase and time fp8bq_row_shards_begin + "
                         "fp8bq_row_shards_finish per group")
    ap.add_argument("--phase", default=None,
                    help="row,col tile phase of each shard for --op shard / shard-rows (default "
                         "bm/2,0: row cuts in the middle of a tile row; shard-rows takes the row "
                         "phase only)")
    ap.add_argument("--per-tensor", action="store_true",
                    help="also time one fp8bq_quantize call per tensor (HIP events per call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-values", type=int, default=0,
                    help="bound the CPU oracle's sample to the first tensors holding about this "
                         "many values (default 0: the whole workload)")
    ap.add_argument("--copies", type=int, default=None,
                    help="rotate this many copies of the inputs and outputs between steps "
                         "(default: 3 for one dense layer, else 1)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records of the default run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--input-sha", action="store_true",
                    help="log the SHA-256 of every input tensor (copies the whole workload to the host)")
    args = ap.parse_args()
    if args.copies is None:
        args.copies = 3 if args.workload == "dense-layer" else 1
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only; --gpus {args.gpus} is not supported "
              "(tiles are independent, so a multi-GPU run would shard rows on tile boundaries "
              "with no exchange)", file=sys.stderr)
        sys.exit(2)

    import ctypes

    import torch

    import fp8_blockwise_weight_amd as fq

    _build.ensure_built()  # load the build of these sources; rebuild if it is of others
    lib_sha = _build.built_sha()
    log(f"libfp8bq.so built from sources {lib_sha}")
    lib = fq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    block = tuple(int(v) for v in args.block.split(",")) if args.block else None
    groups, (bm, bn), desc = build_workload(args.workload, dev, block)
    from fp8_blockwise_weight_amd import workloads as wl

    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    prep = Prepared(lib, groups, bm, bn, dev, sptr, copies=args.copies)
    keep, total_bytes, n_elems, n_tensors = prep.keep, prep.bytes_per_step, prep.elements, prep.tensors
    if args.input_sha:
        for (xs, _), specs in zip(keep, groups):
            for x, sp in zip(xs, specs):
                log(f"input sha256 {sp.name} {sp.M}x{sp.N} {tensor_sha256(x)}")

    # the shard and stream operations time their own calls on the inputs alone
    if args.op == "shard":
        time_shard(lib, keep, groups, bm, bn, args, stream, sptr, desc)
        return
    if args.op == "shard-rows":
        time_row_shards(lib, keep, groups, bm, bn, args, sptr, desc)
        return
    if args.op == "stream":
        time_stream(keep, groups, bm, bn, args, desc)
        return

    ms_per_step, ev_ms = prep.time(args.steps, args.warmup, stream)
    launches = prep.launches
    mean_launch_ms = sum(ev_ms) / len(ev_ms) / launches
    bytes_per_launch = total_bytes / launches
    achieved = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"steps {args.steps}: wall {ms_per_step:.3f} ms/step, events mean {sum(ev_ms) / len(ev_ms):.3f} "
        f"min {min(ev_ms):.3f} max {max(ev_ms):.3f} ms; {value:.1f} GB/s = {100 * value / HBM_PEAK_GBS:.1f}% of peak")

    if args.calibrate_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters
        # calibrate the quantizer's counters (bytes per counted KiB).
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 1 GiB device-to-device")

    if args.op != "quantize":
        time_dequant(lib, keep, groups, bm, bn, args, stream, sptr, desc)
        return

    per_tensor = None
    if args.per_tensor:
        per_tensor = time_per_tensor(lib, keep, groups, bm, bn, stream, sptr)

    traffic = committed_traffic() if args.workload == "dense" else None
    kind = {(128, 128): "kT128", (64, 64): "kT64", (1, 128): "kR128"}.get((bm, bn), "kGeneral")
    flat = kind == "kR128" and all(sp.N % 128 == 0 for specs in groups for sp in specs)
    # the library's choice of the wide [128,128] / [64,64] unit, per launch:
    # every width a multiple of 512 and at least 8192 wide units (the label only)
    if kind in ("kT128", "kT64") and all(
            all(sp.N % 512 == 0 for sp in specs)
            and sum(-(-sp.M // bm) * (sp.N // 512) for sp in specs) >= 8192 for specs in groups):
        kind += "W"
    label, kernels = call_kernels(max(groups, key=len), bm, bn, kind, flat)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": f"{label} ({'one call' if launches == 1 else f'{launches} calls'} per step, "
                  f"{'one kernel launch' if kernels == 1 else f'{kernels} kernel launches'} per call)",
        "bytes_per_launch": bytes_per_launch,
        "mean_launch_ms": round(mean_launch_ms, 4),
        "median_launch_ms": round(sorted(ev_ms)[len(ev_ms) // 2] / launches, 4),
        "min_launch_ms": round(min(ev_ms) / launches, 4),
    }

    cpu = None
    xs_all = None
    if not args.no_cpu_baseline:
        xs_all = [x for xs, _ in keep for x in xs]
        sp_all = [sp for specs in groups for sp in specs]
        take, n = len(sp_all), 0
        if args.cpu_values:
            take = 0
            while take < len(sp_all) and n < args.cpu_values:
                n += sp_all[take].M * sp_all[take].N
                take += 1
        cpu = cpu_baseline(xs_all[:take], sp_all[:take], bm, bn, whole=take == len(sp_all))

    configs = None
    if args.workload == "dense" and args.block is None and not args.no_configs:
        del keep, xs_all, prep
        torch.cuda.empty_cache()
        configs = config_records(lib, dev, sptr, stream, args.steps, args.warmup)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "tensors": n_tensors,
            "elements": n_elems,
            "block": [bm, bn],
            "launches_per_step": launches,
            "algorithmic_bytes_per_step": total_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "lib_sha": lib_sha,
    }
    if configs is not None:
        out["configs"] = configs
    if per_tensor is not None:
        out["per_tensor"] = per_tensor
    print(json.dumps(out), flush=True)


def time_dequant(lib, keep, groups, bm, bn, args, stream, sptr, desc):
    """Dequantize every tensor of the (already quantized) workload, one
    fp8bq_dequantize_many call per group of the workload (the groups the
    quantizer was called with); report output GB/s and % of peak."""
    import torch

    import fp8_blockwise_weight_amd as fq

    f32 = args.op == "dequant-f32"
    esize = 4 if f32 else 2
    items = []   # (table, count) per call
    keep_out = []
    nbytes = 0
    for (xs, outs), specs in zip(keep, groups):
        table = (fq.DqEntry * len(xs))()
        for i, (x, (q, s), sp) in enumerate(zip(xs, outs, specs)):
            o = torch.empty(x.shape, dtype=torch.float32 if f32 else torch.bfloat16, device=x.device)
            keep_out.append(o)
            table[i] = fq.DqEntry(q.data_ptr(), s.data_ptr(), o.data_ptr(), sp.M, sp.N)
            nbytes += sp.M * sp.N * (1 + esize) + 4 * -(-sp.M // bm) * -(-sp.N // bn)
        items.append((table, len(xs)))

    def step():
        for table, count in items:
            st = lib.fp8bq_dequantize_many(table, count, bm, bn, 0 if f32 else 1, sptr)
            if st != 0:
                raise RuntimeError(f"fp8bq_dequantize_many failed: {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    ev = a.elapsed_time(b) / args.steps
    log(f"{args.op}: {len(items)} calls/step, wall {ms:.3f} ms/step (events {ev:.3f}); "
        f"{gbs:.1f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of peak")
    print(json.dumps({"op": args.op, "workload": desc, "calls_per_step": len(items),
                      "bytes_per_step": nbytes, "ms_per_step": round(ms, 4),
                      "GBps": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}),
          flush=True)


def time_shard(lib, keep, groups, bm, bn, args, stream, sptr, desc):
    """Every tensor of the workload as a shard at a tile phase: per group of
    the workload, fp8bq_tile_amax_many (the shards' partial maxima; the
    exchange between shards would sit here) then fp8bq_quantize_amax_many
    with the maxima turned into the scales in place.  Reports GB/s of the
    bytes the two passes move (x read twice, q written, maxima and scales)
    and of the quantizer's algorithmic bytes."""
    import torch

    import fp8_blockwise_weight_amd as fq

    rp, cp = (int(v) for v in args.phase.split(",")) if args.phase else (bm // 2, 0)
    tables = []
    hold = []
    moved = algorithmic = 0
    for (xs, outs), specs in zip(keep, groups):
        arr = (fq.ShardEntry * len(xs))()
        for e, x, (q, _), sp in zip(arr, xs, outs, specs):
            tm, tn = fq.local_grid(sp.M, sp.N, bm, bn, (rp, cp))
            a = torch.empty((tm, tn), dtype=torch.float32, device=x.device)
            hold.append(a)
            e.x, e.q, e.amax, e.scale_inv = x.data_ptr(), q.data_ptr(), a.data_ptr(), a.data_ptr()
            e.M, e.N, e.row_phase, e.col_phase = sp.M, sp.N, rp, cp
            moved += 5 * sp.M * sp.N + 3 * 4 * tm * tn
            algorithmic += 3 * sp.M * sp.N + 4 * tm * tn
        tables.append((arr, len(xs)))

    def step():
        for arr, n in tables:
            st = lib.fp8bq_tile_amax_many(arr, n, bm, bn, sptr)
            if st == 0:
                st = lib.fp8bq_quantize_amax_many(arr, n, bm, bn, sptr)
            if st != 0:
                raise RuntimeError(f"shard path failed: {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / args.steps
    gbs = moved / (ms * 1e-3) / 1e9
    alg = algorithmic / (ms * 1e-3) / 1e9
    log(f"shard at phase ({rp},{cp}): {2 * len(tables)} grouped calls/step, wall {ms:.3f} ms/step; "
        f"{gbs:.1f} GB/s moved = {100 * gbs / HBM_PEAK_GBS:.1f}% of peak, "
        f"{alg:.1f} GB/s algorithmic = {100 * alg / HBM_PEAK_GBS:.1f}%")
    print(json.dumps({"op": "shard", "workload": desc, "phase": [rp, cp],
                      "calls_per_step": 2 * len(tables), "bytes_moved_per_step": moved,
                      "algorithmic_bytes_per_step": algorithmic, "ms_per_step": round(ms, 4),
                      "GBps_moved": round(gbs, 1), "pct_of_hbm_peak_moved": round(100 * gbs / HBM_PEAK_GBS, 2),
                      "GBps_algorithmic": round(alg, 1),
                      "pct_of_hbm_peak_algorithmic": round(100 * alg / HBM_PEAK_GBS, 2)}), flush=True)


def time_row_shards(lib, keep, groups, bm, bn, args, sptr, desc):
    """Every tensor as a row shard (whole rows) at a tile-row phase: per
    group of the workload, fp8bq_row_shards_begin (the edge rows' partial
    maxima, then the whole tile rows between them in one pass; the exchange
    between shards would follow) and fp8bq_row_shards_finish (the edge rows
    with their maxima).  Reports GB/s of the quantizer's algorithmic bytes
    and of the bytes the calls move (edge rows read twice)."""
    import torch

    import fp8_blockwise_weight_amd as fq

    rp = int(args.phase.split(",")[0]) if args.phase else bm // 2
    tables = []
    hold = []
    moved = algorithmic = 0
    for (xs, outs), specs in zip(keep, groups):
        arr = (fq.RowShardEntry * len(xs))()
        for e, x, (q, _), sp in zip(arr, xs, outs, specs):
            tm, tn = fq.local_grid(sp.M, sp.N, bm, bn, (rp, 0))
            s = torch.empty((tm, tn), dtype=torch.float32, device=x.device)
            hold.append(s)
            top, bottom = fq.row_shard_edges(sp.M, bm, rp)
            e.x, e.q, e.scale_inv, e.M, e.N, e.row_phase = x.data_ptr(), q.data_ptr(), s.data_ptr(), sp.M, sp.N, rp
            e.top_amax = s[0].data_ptr() if top else None
            e.bottom_amax = s[tm - 1].data_ptr() if bottom else None
            edge = (top + bottom) * sp.N
            moved += 3 * sp.M * sp.N + 2 * edge + 4 * tm * tn + 8 * ((top > 0) + (bottom > 0)) * tn
            algorithmic += 3 * sp.M * sp.N + 4 * tm * tn
        need = int(lib.fp8bq_many_workspace_bytes(len(xs)))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=keep[0][0][0].device)
        hold.append(ws)
        tables.append((arr, len(xs), ws, need))

    def step():
        for arr, n, ws, need in tables:
            st = lib.fp8bq_row_shards_begin(arr, n, bm, bn, ws.data_ptr(), need, None, sptr)
            if st == 0:
                st = lib.fp8bq_row_shards_finish(arr, n, bm, bn, sptr)
            if st != 0:
                raise RuntimeError(f"row-shard path failed: {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / args.steps
    gbs = moved / (ms * 1e-3) / 1e9
    alg = algorithmic / (ms * 1e-3) / 1e9
    log(f"row shards at row phase {rp}: {2 * len(tables)} calls/step, wall {ms:.3f} ms/step; "
        f"{alg:.1f} GB/s algorithmic = {100 * alg / HBM_PEAK_GBS:.1f}% of peak, "
        f"{gbs:.1f} GB/s moved = {100 * gbs / HBM_PEAK_GBS:.1f}%")
    print(json.dumps({"op": "shard-rows", "workload": desc, "row_phase": rp,
                      "calls_per_step": 2 * len(tables), "bytes_moved_per_step": moved,
                      "algorithmic_bytes_per_step": algorithmic, "ms_per_step": round(ms, 4),
                      "GBps_algorithmic": round(alg, 1),
                      "pct_of_hbm_peak_algorithmic": round(100 * alg / HBM_PEAK_GBS, 2),
                      "GBps_moved": round(gbs, 1),
                      "pct_of_hbm_peak_moved": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def time_stream(keep, groups, bm, bn, args, desc):
    """stream.quant_weights over the workload's weights in model order, with a
    1-D norm weight (passed through) before each layer's attention and MLP
    blocks, as a decoder's named parameters come; every yielded pair is
    consumed.  Reports algorithmic GB/s of the FP8 weights, wall clock."""
    import torch

    import fp8_blockwise_weight_amd as fq
    from fp8_blockwise_weight_amd.stream import quant_weights

    dev = torch.device("cuda:0")
    pairs = []
    nbytes = 0
    layer = None
    for (xs, _), specs in zip(keep, groups):
        for x, sp in zip(xs, specs):
            prefix = ".".join(sp.name.split(".")[:2])      # "layers.<i>"
            if prefix != layer:
                layer = prefix
                pairs.append((f"{layer}.input_layernorm.weight",
                              torch.ones(x.shape[1], dtype=torch.bfloat16, device=dev)))
            if sp.name.endswith("gate_proj"):
                pairs.append((f"{layer}.post_attention_layernorm.weight",
                              torch.ones(x.shape[1], dtype=torch.bfloat16, device=dev)))
            pairs.append((f"{sp.name}.weight", x))
            nbytes += algorithmic_bytes(sp.M, sp.N, bm, bn)
    fq.load_library()

    def step():
        n = 0
        for _name, _t in quant_weights(pairs, (bm, bn)):
            n += 1
        return n

    for _ in range(args.warmup):
        yielded = step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        yielded = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"stream: {len(pairs)} pairs in, {yielded} out per step, wall {ms:.3f} ms/step; "
        f"{gbs:.1f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of peak")
    print(json.dumps({"op": "stream", "workload": desc, "pairs_in": len(pairs), "pairs_out": yielded,
                      "bytes_per_step": nbytes, "ms_per_step": round(ms, 4), "GBps": round(gbs, 1),
                      "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def time_per_tensor(lib, keep, groups, bm, bn, stream, sptr, reps=3):
    """One fp8bq_quantize launch per tensor, HIP events around each call.
    Returns GB/s per tensor shape (mean over tensors of that shape) and the
    end-to-end rate of the per-tensor loop."""
    import torch

    calls = []
    for (xs, outs), specs in zip(keep, groups):
        for x, (q, s), sp in zip(xs, outs, specs):
            calls.append((sp, x, q, s))
    for sp, x, q, s in calls[:8]:
        lib.fp8bq_quantize(x.data_ptr(), sp.M, sp.N, bm, bn, q.data_ptr(), s.data_ptr(), sptr)
    torch.cuda.synchronize()
    by_shape = {}
    t0 = time.perf_counter()
    for _ in range(reps):
        evs = []
        for sp, x, q, s in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = lib.fp8bq_quantize(x.data_ptr(), sp.M, sp.N, bm, bn, q.data_ptr(), s.data_ptr(), sptr)
            b.record(stream)
            if st != 0:
                raise RuntimeError(f"fp8bq_quantize failed: {st}")
            evs.append((sp, a, b))
        torch.cuda.synchronize()
        for sp, a, b in evs:
            key = f"{sp.name.split('.')[-1]} {sp.M}x{sp.N}"
            by_shape.setdefault(key, []).append(algorithmic_bytes(sp.M, sp.N, bm, bn) / (a.elapsed_time(b) * 1e-3) / 1e9)
    wall = (time.perf_counter() - t0) / reps
    total = sum(algorithmic_bytes(sp.M, sp.N, bm, bn) for sp, *_ in calls)
    res = {k: round(sum(v) / len(v), 1) for k, v in by_shape.items()}
    res["loop_of_single_calls_GBps"] = round(total / wall / 1e9, 1)
    log("per-tensor single calls (GB/s): " + json.dumps(res))
    return res


def tensor_sha256(x):
    """SHA-256 of a tensor's bytes (copied to the host)."""
    import numpy as np
    import torch

    return hashlib.sha256(x.view(torch.int16).cpu().numpy().view(np.uint8).tobytes()).hexdigest()


def cpu_baseline(xs, specs, bm, bn, whole=True):
    """The CPU oracle as it is, on the host's cores: a pool of worker
    processes (one per core this process may use, at most 16) quantizes the
    sample one slab of whole tile rows at a time, from the BF16 bits in
    shared host memory to the codes and scales.  The copy of the inputs to
    the host is not timed."""
    import numpy as np
    import torch

    from oracle.pool import OraclePool

    nbytes = sum(algorithmic_bytes(sp.M, sp.N, bm, bn) for sp in specs)
    nel = sum(sp.M * sp.N for sp in specs)
    arena = sum(3 * sp.M * sp.N + 4 * -(-sp.M // bm) * -(-sp.N // bn) + 1024 for sp in specs)
    digest = hashlib.sha256()
    with OraclePool(arena) as pool:
        items = []
        t0 = time.perf_counter()
        for i, (x, sp) in enumerate(zip(xs, specs)):
            xa = pool.arena.array((sp.M, sp.N), np.uint16)
            torch.from_numpy(xa.view(np.int16)).copy_(x.view(torch.int16))
            qa = pool.arena.array((sp.M, sp.N), np.uint8)
            sa = pool.arena.array((-(-sp.M // bm), -(-sp.N // bn)), np.float32)
            items.append((i, xa, qa, sa))
        log(f"cpu oracle: {len(items)} inputs copied to shared host memory in {time.perf_counter() - t0:.1f}s")
        dt = pool.quantize(items, bm, bn)
        workers = pool.workers
        for (_, xa, _, _), sp in zip(items, specs[:4]):
            one = hashlib.sha256(xa.tobytes()).hexdigest()
            digest.update(bytes.fromhex(one))
            log(f"input sha256 {sp.name} {sp.M}x{sp.N} {one}")
        del items, xa, qa, sa
    log(f"cpu oracle: {len(specs)} tensors, {nel / 1e6:.1f} M values in {dt:.1f}s on {workers} processes")
    what = "the whole benchmarked workload" if whole else "the first tensors of the benchmarked workload"
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{what}: {len(specs)} tensors, {nel} values; the numpy oracle in {workers} worker "
                  f"processes (one per available host core, at most 16), {dt:.1f} s wall from BF16 bits "
                  "in host memory to codes and scales",
        "sample_sha256": digest.hexdigest(),
        "sample_sha256_covers": f"the first {min(4, len(specs))} inputs",
    }


if __name__ == "__main__":
    main()
