"""bench.py keeps its output contract: one JSON line with the required keys
(GPU), and a refusal with a message for more than one GPU (CPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                         timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line(gpu_lib):
    """A short run on one dense layer: the last stdout line is the JSON
    record with every key the contract names, consistent with itself."""
    print("bench.py --workload dense-layer --steps 3 --warmup 1", flush=True)
    res = subprocess.run([sys.executable, BENCH, "--workload", "dense-layer", "--steps", "3",
                          "--warmup", "1", "--cpu-values", "1"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "GB/s" and rec["higher_is_better"] is True
    assert "workload" in rec["config"] and rec["config"]["tensors"] == 7
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1
    cpu = rec["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert 1 <= cpu["cores"] <= 16 and "1 tensors" in cpu["sample"]
    sys.path.insert(0, ROOT)
    from fp8_blockwise_weight_amd import build

    assert rec["lib_sha"] == build.built_sha() == build.source_sha()
    assert "configs" not in rec          # only the default run measures the other sets
    # value = algorithmic bytes / wall time per step
    want = rec["config"]["algorithmic_bytes_per_step"] / (rec["ms_per_step"] * 1e-3) / 1e9
    assert abs(rec["value"] - want) / want < 1e-3


@pytest.mark.gpu
def test_bench_shard_mode(gpu_lib):
    """--op shard on one dense layer: every tensor as a shard at a tile phase
    through the grouped tile_amax and quantize_amax calls; the record's byte
    counts follow the two-pass formula."""
    print("bench.py --workload dense-layer --op shard --phase 64,0", flush=True)
    res = subprocess.run([sys.executable, BENCH, "--workload", "dense-layer", "--op", "shard",
                          "--phase", "64,0", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["op"] == "shard" and rec["phase"] == [64, 0] and rec["calls_per_step"] == 2
    sys.path.insert(0, ROOT)
    from fp8_blockwise_weight_amd import workloads as wl

    moved = alg = 0
    for sp in wl.c2():
        tm, tn = -(-(64 + sp.M) // 128), -(-sp.N // 128)
        moved += 5 * sp.M * sp.N + 12 * tm * tn
        alg += 3 * sp.M * sp.N + 4 * tm * tn
    assert rec["bytes_moved_per_step"] == moved and rec["algorithmic_bytes_per_step"] == alg
    assert 0 < rec["pct_of_hbm_peak_moved"] < 100


@pytest.mark.gpu
def test_bench_row_shard_mode(gpu_lib):
    """--op shard-rows on one dense layer: every tensor as a row shard at row
    phase 64 through fp8bq_row_shards_begin / _finish; the record's byte
    counts follow the edge-rows formula."""
    print("bench.py --workload dense-layer --op shard-rows --phase 64", flush=True)
    res = subprocess.run([sys.executable, BENCH, "--workload", "dense-layer", "--op", "shard-rows",
                          "--phase", "64", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["op"] == "shard-rows" and rec["row_phase"] == 64 and rec["calls_per_step"] == 2
    sys.path.insert(0, ROOT)
    from fp8_blockwise_weight_amd import workloads as wl

    moved = alg = 0
    for sp in wl.c2():
        tm, tn = -(-(64 + sp.M) // 128), -(-sp.N // 128)
        edge = 64 + (sp.M - 64) % 128                      # 64 top rows, the rest of the last tile row
        moved += 3 * sp.M * sp.N + 2 * edge * sp.N + 4 * tm * tn + 16 * tn
        alg += 3 * sp.M * sp.N + 4 * tm * tn
    assert rec["bytes_moved_per_step"] == moved and rec["algorithmic_bytes_per_step"] == alg
    assert 0 < rec["pct_of_hbm_peak_algorithmic"] < 100


@pytest.mark.gpu
def test_bench_stream_mode(gpu_lib):
    """--op stream on one dense layer: every weight and the norms in model
    order through quant_weights; the record counts the pairs in and out
    (two out per FP8 weight) and the weights' algorithmic bytes."""
    print("bench.py --workload dense-layer --op stream", flush=True)
    res = subprocess.run([sys.executable, BENCH, "--workload", "dense-layer", "--op", "stream",
                          "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["op"] == "stream"
    sys.path.insert(0, ROOT)
    from fp8_blockwise_weight_amd import workloads as wl

    specs = wl.c2()
    n_fp8 = len(specs)
    assert rec["pairs_out"] == rec["pairs_in"] + n_fp8
    assert rec["bytes_per_step"] == sum(3 * sp.M * sp.N + 4 * (-(-sp.M // 128)) * (-(-sp.N // 128))
                                        for sp in specs)
    assert 0 < rec["pct_of_hbm_peak"] < 100


def test_kernel_fingerprint_ignores_comments_only():
    """The counter record is tied to the kernels' code: comment and layout
    edits keep the fingerprint, code edits change it."""
    sys.path.insert(0, ROOT)
    import bench

    base = 'int f(int a) {  // twice\n  return a * 2; /* doubled */ }\nconst char* s = "//x";\n'
    same = '// header\nint f(int a) {\n    return a * 2;\n}\nconst char* s = "//x";  /* note */\n'
    other = 'int f(int a) { return a * 3; }\nconst char* s = "//x";\n'
    assert bench._code_only(base) == bench._code_only(same)
    assert bench._code_only(base) != bench._code_only(other)
    assert bench._code_only('const char* s = "//x";') == 'const char* s = "//x";'
    assert len(bench.kernel_sha()) == 16


def test_call_kernels_label_mirrors_library_choice():
    """The bench's label of what one grouped call launches follows the
    library's rules: the four-tile [128,128] kernel for the dense set, the
    register-resident pair for one-tile lists within capacity, the two-pass
    kernels beyond it."""
    import bench
    from fp8_blockwise_weight_amd import workloads as wl

    assert bench.call_kernels(wl.c3(), 128, 128, "kT128W", False) == (
        "fp8bq::quantize_group_args<kT128W,512>", 1)
    label, k = bench.call_kernels(wl.c3(), 12288, 12288, "kGeneral", False)
    assert "resident_group<256>" in label and k == 2
    label, k = bench.call_kernels(wl.c2()[:1], 4096, 4096, "kGeneral", False)
    assert "resident_quant" in label and k == 2
    vocab = [s for s in wl.c5() if s.M == 151937]
    assert bench.call_kernels(vocab, 151937, 4096, "kGeneral", False)[1] == 3
    assert bench.RESIDENT_CAPACITY == 12288 * 4096
