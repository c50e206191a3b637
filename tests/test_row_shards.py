"""Row shards with the exchange confined to shared tile rows
(fp8bq_row_shard_edges, fp8bq_row_shards_begin / _finish).

CPU: the edge split against a brute-force reading of which rows lie in
tile rows a shard holds whole.  GPU: matrices cut into row shards anywhere
(inside tile rows, shards thinner than a tile row, hundreds of shards),
quantized shard by shard with the edge maxima exchanged between the shards
that share a tile row, reassembled: every byte and scale equals quantizing
the whole matrix, on the GPU and in the oracle."""

import numpy as np
import pytest
import torch

import fp8_blockwise_weight_amd as fq


def _edges_brute(M, bm, rp):
    """Group the shard's rows by the tile row they fall in; rows of tile rows
    the shard does not hold whole are edges: the first group when the shard
    starts inside a tile row, the last group when it ends inside one."""
    groups = {}
    for i in range(M):
        groups.setdefault((rp + i) // bm, []).append(i)
    order = sorted(groups)
    whole = {t for t in order if len(groups[t]) == bm}
    top = len(groups[order[0]]) if order and rp > 0 else 0
    bottom = 0
    if order and (rp + M) % bm != 0 and not (rp > 0 and len(order) == 1):
        bottom = len(groups[order[-1]])
    inner = [t for t in order if t in whole and not (top and t == order[0])]
    assert sum(len(groups[t]) for t in inner) == M - top - bottom
    return top, bottom


def test_row_shard_edges_brute_force():
    for bm in (1, 2, 3, 5, 8, 128):
        for rp in range(bm):
            for M in range(0, 3 * bm + 3):
                assert fq.row_shard_edges(M, bm, rp) == _edges_brute(M, bm, rp), (M, bm, rp)


# ------------------------------------------------------------------ GPU

DEV = "cuda:0"


def _exchange(spans, bm):
    """The max-exchange between shards sharing a tile row, on one GPU.
    ``spans`` holds each shard's (first row, rows) in the full matrix."""

    def run(edges):
        groups = {}
        for (r0, M), (top, bottom) in zip(spans, edges):
            if top is not None:
                groups.setdefault(r0 // bm, []).append(top)
            if bottom is not None:
                groups.setdefault((r0 + M - 1) // bm, []).append(bottom)
        for parts in groups.values():
            full = parts[0].clone()
            for a in parts[1:]:
                full = torch.maximum(full, a)
            for a in parts:
                a.copy_(full)

    return run


def _assemble(x, outs, spans, bm, bn):
    """Whole-matrix q and scales from the shards' outputs; scale rows that
    several shards hold must agree bit for bit."""
    M, N = x.shape
    TM, TN = fq.scale_shape(M, N, bm, bn)
    q = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    s = torch.full((TM, TN), float("nan"), dtype=torch.float32, device=DEV)
    seen = torch.zeros(TM, dtype=torch.bool)
    for (r0, rows), (qi, si) in zip(spans, outs):
        q[r0:r0 + rows] = qi.view(torch.uint8)
        if rows == 0:
            continue
        t0 = r0 // bm
        for k in range(si.shape[0]):
            if seen[t0 + k]:
                assert torch.equal(s[t0 + k].view(torch.int32), si[k].view(torch.int32)), (r0, k)
            s[t0 + k] = si[k]
            seen[t0 + k] = True
    assert bool(seen.all())
    return q, s


def _cut(M, cuts):
    bounds = [0] + sorted(set(c for c in cuts if 0 < c < M)) + [M]
    return [(a, b - a) for a, b in zip(bounds, bounds[1:])]


# the last three: rows not 16-byte aligned (N % 8 != 0) and tile columns off
# 8-element boundaries, so edges and whole tile rows take the element-wise
# and two-pass kernels
CASES = [(1000, 3000, (128, 128)), (1536, 2048, (128, 128)), (4097, 1024, (64, 64)),
         (300, 640, (1, 128)), (777, 520, (32, 96)), (99, 37, (5, 3)), (3000, 2000, (1024, 1024)),
         (300, 77, (16, 16)), (500, 1000, (100, 100)), (700, 1200, (256, 300))]


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,block", CASES, ids=[f"{m}x{n}-{b[0]}x{b[1]}" for m, n, b in CASES])
def test_row_shards_equal_whole(gpu_lib, M, N, block):
    from gpu_helpers import assert_matches_oracle

    bm, bn = block
    g = torch.Generator(device=DEV).manual_seed(M + N)
    rng = np.random.default_rng(M * 7 + N)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    x[min(M - 1, 3 * bm // 2)] *= 40          # an outlier row inside a shared tile row
    q_ref, s_ref = fq.quantize(x, block)
    cut_sets = [list(rng.integers(1, M, rng.integers(1, 6))) for _ in range(3)]
    cut_sets.append([bm + 2, bm + 3, bm + 9, 2 * bm + 1])   # shards thinner than a tile row
    cut_sets.append([])                                      # the whole matrix, phase 0
    for cuts in cut_sets:
        spans = _cut(M, [int(c) for c in cuts])
        print("row shards", M, N, block, [r0 for r0, _ in spans], flush=True)
        shards = [x[r0:r0 + rows] for r0, rows in spans]
        outs = fq.quantize_row_shards(shards, block, [r0 % bm for r0, _ in spans],
                                      exchange=_exchange(spans, bm))
        for (r0, rows), (qi, si) in zip(spans, outs):
            assert tuple(qi.shape) == (rows, N)
            assert tuple(si.shape) == fq.local_grid(rows, N, bm, bn, (r0 % bm, 0))
        q, s = _assemble(x, outs, spans, bm, bn)
        assert torch.equal(q, q_ref.view(torch.uint8)), cuts
        assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32)), cuts
    assert_matches_oracle(x, q_ref, s_ref, bm, bn, f"row shards {M}x{N} {block}")


@pytest.mark.gpu
def test_row_shards_many_and_side_stream(gpu_lib):
    """600 shards (the whole-tile parts' table goes through the workspace),
    with the exchange on a second stream that waits for the maxima event and
    the finishing call ordered after it; also shards of zero rows."""
    from gpu_helpers import assert_matches_oracle

    bm, bn = 128, 128
    M, N = 600 * 150, 256
    g = torch.Generator(device=DEV).manual_seed(3)
    rng = np.random.default_rng(3)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.03).to(torch.bfloat16)
    cuts = sorted(set(int(c) for c in rng.integers(1, M, 599)))
    spans = _cut(M, cuts)
    spans.insert(5, (spans[5][0], 0))                       # an empty shard between two others
    shards = [x[r0:r0 + rows] for r0, rows in spans]
    print("row shards, side stream", len(shards), flush=True)
    ev, done = torch.cuda.Event(), torch.cuda.Event()
    state = fq.row_shards_begin(shards, (bm, bn), [r0 % bm for r0, _ in spans], maxima_event=ev)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        side.wait_event(ev)
        _exchange(spans, bm)(state.edges)
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    outs = fq.row_shards_finish(state)
    torch.cuda.synchronize()
    assert tuple(outs[5][0].shape) == (0, N) and tuple(outs[5][1].shape) == (0, 2)
    q, s = _assemble(x, outs, spans, bm, bn)
    q_ref, s_ref = fq.quantize(x, (bm, bn))
    assert torch.equal(q, q_ref.view(torch.uint8))
    assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32))
    assert_matches_oracle(x, q_ref, s_ref, bm, bn, "600 row shards")


@pytest.mark.gpu
def test_row_shards_graph_capture(gpu_lib):
    """fp8bq_row_shards_begin, a max-exchange in torch and
    fp8bq_row_shards_finish captured in one HIP graph over 600 row shards
    (the whole-tile parts take launches with the table in the kernel
    arguments under capture): every replay, with the input rescaled eagerly
    in between, equals the eager whole-matrix quantization."""
    import ctypes

    bm, bn = 128, 128
    M, N = 600 * 150, 256
    g = torch.Generator(device=DEV).manual_seed(17)
    rng = np.random.default_rng(17)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.03).to(torch.bfloat16)
    spans = _cut(M, [int(c) for c in rng.integers(1, M, 599)])
    n = len(spans)
    table = (fq.RowShardEntry * n)()
    outs, edges = [], []
    for e, (r0, rows) in zip(table, spans):
        rp = r0 % bm
        TMl, TN = fq.local_grid(rows, N, bm, bn, (rp, 0))
        top, bottom = fq.row_shard_edges(rows, bm, rp)
        q = torch.empty((rows, N), dtype=torch.uint8, device=DEV)
        s = torch.empty((TMl, TN), dtype=torch.float32, device=DEV)
        e.x, e.q, e.scale_inv, e.M, e.N, e.row_phase = x[r0].data_ptr(), q.data_ptr(), s.data_ptr(), rows, N, rp
        e.top_amax = s[0].data_ptr() if top else None
        e.bottom_amax = s[TMl - 1].data_ptr() if bottom else None
        outs.append((q, s))
        edges.append((s[0] if top else None, s[TMl - 1] if bottom else None))
    lib = gpu_lib.load_library()
    need = int(lib.fp8bq_many_workspace_bytes(n))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    exchange = _exchange(spans, bm)

    def calls():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.fp8bq_row_shards_begin(table, n, bm, bn, ws.data_ptr(), need, None, st) == 0
        exchange(edges)
        assert lib.fp8bq_row_shards_finish(table, n, bm, bn, st) == 0

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
        print("row-shard graph replay", rep, flush=True)
        x.mul_(2.0 if rep % 2 else 0.5)                    # exact: powers of two
        for q, s in outs:
            q.fill_(0xA5)
            s.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        q_ref, s_ref = fq.quantize(x, (bm, bn))
        q, s = _assemble(x, [(q.view(torch.float8_e4m3fn), s) for q, s in outs], spans, bm, bn)
        assert torch.equal(q, q_ref.view(torch.uint8)), rep
        assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32)), rep
