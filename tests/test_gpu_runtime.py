"""Runtime behaviour on the GPU: HIP-graph capture and replay, non-default
streams, and concurrent calls from several host threads."""

import threading

import numpy as np
import pytest
import torch

import fp8_blockwise_weight_amd as fq
from fp8_blockwise_weight_amd import workloads as wl
from gpu_helpers import assert_matches_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("block", [(128, 128), (1, 128), (4096, 4096)])
def test_graph_capture_replays_match_eager(gpu_lib, block):
    """A grouped call (table in the kernel arguments; for the 4096x4096
    block, the two-pass large-tile kernels) captured in a HIP graph: every
    replay, with eager work and synchronizations in between, equals an
    eager call on the same inputs."""
    specs = wl.c2()[:3] + wl.c4_layer(0)[:5]
    xs = [wl.materialize(sp, DEV) for sp in specs]
    outs = [(torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=DEV),
             torch.empty(fq.scale_shape(*x.shape, *block), dtype=torch.float32, device=DEV))
            for x in xs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.quantize_many(xs, block, outputs=outs)          # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fq.quantize_many(xs, block, outputs=outs)
    torch.cuda.synchronize()
    g = torch.Generator(device=DEV).manual_seed(3)
    for rep in range(4):
        _say("replay", block, rep)
        for x in xs:                                       # eager work between replays
            x.mul_(torch.where(torch.rand(x.shape, generator=g, device=DEV) < 0.5, -1.0, 1.0)
                   .to(torch.bfloat16))
        for q, s in outs:
            q.view(torch.uint8).fill_(0xA5)
            s.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, (q, s) in zip(xs, outs):
            q1, s1 = fq.quantize(x, block)
            assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), (block, rep)
            assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), (block, rep)
    assert_matches_oracle(xs[0], outs[0][0], outs[0][1], *block, "graph replay")


@pytest.mark.parametrize("block", [(128, 128), (64, 64), (1, 128), (5, 3)])
def test_graph_capture_beyond_argument_table(gpu_lib, block):
    """More tensors than the kernel arguments hold (700), captured in a HIP
    graph: under capture the call enqueues several launches of at most 512
    tensors each instead of copying the table into the workspace, and every
    replay, with eager work in between, equals eager single calls."""
    g = torch.Generator(device=DEV).manual_seed(29)
    rng = np.random.default_rng(29)
    xs = []
    for _ in range(700):
        M, N = int(rng.integers(1, 300)), int(rng.choice([8, 64, 136, 256, 264, 7, 99]))
        xs.append((torch.randn((M, N), generator=g, device=DEV) * 0.03).to(torch.bfloat16))
    assert fq.workspace_bytes(len(xs)) > 0
    outs = [(torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=DEV),
             torch.empty(fq.scale_shape(*x.shape, *block), dtype=torch.float32, device=DEV))
            for x in xs]
    ws = torch.empty(fq.workspace_bytes(len(xs)), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.quantize_many(xs, block, outputs=outs, workspace=ws)   # eager: workspace path
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ws.fill_(0x5A)                                         # the graph must never write it
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fq.quantize_many(xs, block, outputs=outs, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        _say("replay beyond the argument table", block, rep)
        for x in xs:                                       # eager work between replays
            x.neg_()
        for q, s in outs:
            q.view(torch.uint8).fill_(0xA5)
            s.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (x, (q, s)) in enumerate(zip(xs, outs)):
            q1, s1 = fq.quantize(x, block)
            assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), (block, rep, i)
            assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), (block, rep, i)
    assert bool((ws == 0x5A).all()), "a captured call copied its table into the workspace"
    for i in (0, 511, 512, 699):
        assert_matches_oracle(xs[i], outs[i][0], outs[i][1], *block, f"graph beyond table [{i}]")


def test_graph_capture_of_grouped_shard_calls(gpu_lib):
    """Grouped shard calls (maxima, then quantize with the maxima converted
    in place) captured in one HIP graph: every replay, with the inputs
    changed eagerly in between, equals the eager calls."""
    import ctypes

    g = torch.Generator(device=DEV).manual_seed(59)
    shapes = [(300, 520), (1536, 2048), (77, 128), (2048, 768), (5, 8)] * 60   # 300 shards
    xs = [(torch.randn(sh, generator=g, device=DEV) * 0.02).to(torch.bfloat16) for sh in shapes]
    phases = [(64 if i % 2 else 0, 8 * (i % 3)) for i in range(len(xs))]
    block = (128, 128)
    grids = [fq.local_grid(*x.shape, *block, ph) for x, ph in zip(xs, phases)]
    amaxs = [torch.empty(gr, dtype=torch.float32, device=DEV) for gr in grids]
    qs = [torch.empty(x.shape, dtype=torch.uint8, device=DEV) for x in xs]
    arr = (fq.ShardEntry * len(xs))()
    for e, x, ph, a, q in zip(arr, xs, phases, amaxs, qs):
        e.x, e.q, e.amax, e.scale_inv = x.data_ptr(), q.data_ptr(), a.data_ptr(), a.data_ptr()
        e.M, e.N = x.shape
        e.row_phase, e.col_phase = ph
    lib = gpu_lib.load_library()

    def calls():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.fp8bq_tile_amax_many(arr, len(xs), *block, st) == 0
        assert lib.fp8bq_quantize_amax_many(arr, len(xs), *block, st) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                            # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        _say("shard graph replay", rep)
        for x in xs:
            x.mul_(2.0 if rep % 2 else 0.5)                # exact: powers of two
        for q, a in zip(qs, amaxs):
            q.fill_(0xA5)
            a.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, ph, a, q in zip(xs, phases, amaxs, qs):
            a1 = fq.tile_amax(x, block, ph)
            q1, s1 = fq.quantize_with_amax(x, a1, block, ph)
            assert torch.equal(q, q1.view(torch.uint8)), rep
            assert torch.equal(a.view(torch.int32), s1.view(torch.int32)), rep


def test_non_default_streams(gpu_lib):
    """Work is enqueued on the caller's current stream and ordered with it."""
    x = wl.materialize(wl.c2()[0], DEV)
    q0, s0 = fq.quantize(x, (128, 128))
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        y = x * 2                                          # produced on st
        q1, s1 = fq.quantize(y, (128, 128))                # must see y on st
        xh = fq.dequantize(q1, s1, (128, 128))
    st.synchronize()
    assert torch.equal(q1.view(torch.uint8), q0.view(torch.uint8))   # scaling by 2 is exact
    assert torch.equal(s1, s0 * 2)
    assert xh.shape == x.shape


def test_concurrent_host_threads(gpu_lib):
    """Several host threads, each with its own stream, quantizing different
    weight lists at once (grouped and single calls) give the same bytes as
    one thread doing it alone."""
    lists = [[wl.materialize(sp, DEV) for sp in wl.c4_layer(layer)[:64]] for layer in range(4)]
    ref = [[(q.view(torch.uint8).clone(), s.clone()) for q, s in fq.quantize_many(xs, (128, 128))]
           for xs in lists]
    torch.cuda.synchronize()
    results = [None] * len(lists)
    errors = []

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                got = []
                for _ in range(3):
                    got = fq.quantize_many(lists[i], (128, 128))
                    singles = [fq.quantize(x, (128, 128)) for x in lists[i][:8]]
                st.synchronize()
            results[i] = (got, singles)
        except Exception as exc:  # noqa: BLE001 - reported below
            errors.append(exc)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(lists))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (got, singles) in enumerate(results):
        for (q, s), (qr, sr) in zip(got, ref[i]):
            assert torch.equal(q.view(torch.uint8), qr) and torch.equal(s, sr), i
        for (q, s), (qr, sr) in zip(singles, ref[i][:8]):
            assert torch.equal(q.view(torch.uint8), qr), i


def test_per_tensor_held_in_registers_beside_other_streams(gpu_lib):
    """One-scale-per-tensor lists (persistent launches that hold tensors in
    registers and wait for each other's maxima) on two streams at once, next
    to a [128,128] launch on a third: the launches compete for the CUs, so
    workgroups may not be resident together and some may pass the wait limit
    and compute maxima themselves.  Every byte equals the sequential results,
    with the default limit and with a 20 us limit.  A captured single call
    replays to the same bytes."""
    g = torch.Generator(device=DEV).manual_seed(97)
    lists = [[(torch.randn((2048, 2048), generator=g, device=DEV) * (0.01 * (i + 1))).to(torch.bfloat16)
              for i in range(40)] for _ in range(2)]
    dense = [wl.materialize(sp, DEV) for sp in wl.c2()]
    block = (4096, 4096)
    ref = [[(q.view(torch.uint8).clone(), s.clone()) for q, s in fq.quantize_many(xs, block)] for xs in lists]
    ref_dense = [(q.view(torch.uint8).clone(), s.clone()) for q, s in fq.quantize_many(dense, (128, 128))]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    try:
        for wait_us in (2000, 20):
            _say("concurrent resident lists, wait limit", wait_us)
            fq.set_resident_wait_us(wait_us)
            for rep in range(2):
                got = [None, None]
                for st in streams:
                    st.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(streams[2]):
                    got_dense = fq.quantize_many(dense, (128, 128))
                for i in range(2):
                    with torch.cuda.stream(streams[i]):
                        got[i] = fq.quantize_many(lists[i], block)
                torch.cuda.synchronize()
                for i in range(2):
                    for j, ((q, s), (qr, sr)) in enumerate(zip(got[i], ref[i])):
                        assert torch.equal(q.view(torch.uint8), qr), (wait_us, rep, i, j)
                        assert torch.equal(s.view(torch.int32), sr.view(torch.int32)), (wait_us, rep, i, j)
                for (q, s), (qr, sr) in zip(got_dense, ref_dense):
                    assert torch.equal(q.view(torch.uint8), qr) and torch.equal(s, sr)
    finally:
        fq.set_resident_wait_us(2000)
    # a captured single call (prep + resident kernel), replayed with eager work between
    x = wl.materialize(wl.c2()[0], DEV)                    # 4096x4096: one resident launch
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((1, 1), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.quantize(x, (4096, 4096), out=(q, s))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fq.quantize(x, (4096, 4096), out=(q, s))
    torch.cuda.synchronize()
    for rep in range(3):
        _say("resident graph replay", rep)
        x.mul_(-1.5 if rep % 2 else 0.75)
        q.view(torch.uint8).fill_(0xA5)
        s.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        q1, s1 = fq.quantize(x, (4096, 4096))
        assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), rep
        assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), rep


def test_graph_capture_of_grouped_dequantization(gpu_lib):
    """fp8bq_dequantize_many captured in a HIP graph (table in the kernel
    arguments): every replay, with the codes changed eagerly in between,
    equals single eager calls, for both output types."""
    g = torch.Generator(device=DEV).manual_seed(71)
    xs = [(torch.randn((int(m), int(n)), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
          for m, n in ((300, 512), (1024, 1024), (77, 128), (513, 2048))] * 5
    qs, ss = zip(*fq.quantize_many(xs, (128, 128)))
    qs = [q.view(torch.uint8) for q in qs]
    for dt in (torch.float32, torch.bfloat16):
        outs = [torch.empty(q.shape, dtype=dt, device=DEV) for q in qs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fq.dequantize_many(qs, ss, (128, 128), out_dtype=dt, outs=outs)   # warm-up
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fq.dequantize_many(qs, ss, (128, 128), out_dtype=dt, outs=outs)
        torch.cuda.synchronize()
        for rep in range(3):
            _say("grouped dequant replay", dt, rep)
            for q in qs:
                q.copy_(torch.where(q == 0x7F, q, q ^ 0x80))     # flip signs, keep NaN codes away
            for o in outs:
                o.fill_(-7.0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (q, s, o) in enumerate(zip(qs, ss, outs)):
                one = fq.dequantize(q, s, (128, 128), out_dtype=dt)
                assert torch.equal(o.view(torch.int16), one.view(torch.int16)), (dt, rep, i)


def test_error_reporting_on_device(gpu_lib):
    """Argument errors raise with the library's status text; nothing is
    launched (outputs keep their fill)."""
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    q = torch.full((64, 64), 0x11, dtype=torch.uint8, device=DEV)
    s = torch.full((1, 1), 3.0, device=DEV)
    with pytest.raises(fq.Fp8bqError, match="invalid argument"):
        fq.quantize(x, (64, 64), out=(q.view(64, 64), x[:1, :2].view(torch.float32)))  # scale overlaps x
    torch.cuda.synchronize()
    assert bool((q == 0x11).all()) and float(s[0, 0]) == 3.0
    ws_small = torch.empty(16, dtype=torch.uint8, device=DEV)
    mats = [torch.zeros((8, 8), dtype=torch.bfloat16, device=DEV) for _ in range(600)]
    with pytest.raises(fq.Fp8bqError, match="workspace"):
        fq.quantize_many(mats, (8, 8), workspace=ws_small)
    assert np.isfinite(1.0)
