"""The seeded synthetic workloads (CPU): determinism, shapes and the planted
structure each recipe promises."""

import math

import torch

from fp8_blockwise_weight_amd import workloads as wl


def test_c1_structure_and_determinism():
    (spec,) = wl.c1()
    a = wl.materialize(spec)
    b = wl.materialize(spec)
    assert a.dtype == torch.bfloat16 and a.shape == (256, 256)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    t00 = a[:128, :128].float()
    assert int((t00.abs() == 5.0).sum()) == 8                 # 8 planted +-5.0
    assert torch.all(a[128:, 128:] == 0)                       # the all-zero tile
    rest = torch.cat([a[:128, 128:].reshape(-1), a[128:, :128].reshape(-1)]).float()
    assert 0.015 < float(rest.std()) < 0.025                   # N(0, 0.02)


def test_dense_layer_shapes_and_seeds():
    layer = wl.dense_layer(3)
    assert [(s.M, s.N) for s in layer] == [(M, N) for _, M, N in wl.QWEN3_8B_LAYER]
    assert len({s.seed for s in wl.c3()}) == 252
    assert sum(s.numel for s in wl.c3()) == 6_945_767_424
    assert wl.c2()[0].seed != wl.dense_layer(0)[0].seed        # C2 and C3 draw differently


def test_dense_outliers_distribution():
    sp = wl.TensorSpec("t", 512, 1024, wl.seed_of(9, 0, 0), "dense")
    x = wl.materialize(sp).float()
    big = x.abs() > 0.2                                        # ~10 sigma of N(0,0.02)
    k = round(1e-4 * sp.numel)
    assert 0 < int(big.sum()) <= k                             # outliers are the only large values
    core = x[~big]
    assert 0.018 < float(core.std()) < 0.022


def test_moe_sigmas_and_shapes():
    sig = wl.moe_sigmas(7)
    assert len(sig) == 128 and all(0.01 <= v <= 0.04 for v in sig)
    assert wl.moe_sigmas(7) == sig
    layer = wl.c4_layer(7)
    assert len(layer) == 256
    assert {(s.M, s.N) for s in layer} == {wl.MOE_W13, wl.MOE_DOWN}
    w13, down = layer[10], layer[11]
    assert w13.sigma == down.sigma                             # one sigma per expert
    x = wl.materialize(w13).float()
    assert abs(float(x.std()) - w13.sigma) < 0.05 * w13.sigma


def test_ragged_zero_rows_and_mixture():
    sp = wl.TensorSpec("r", 1000, 512, wl.seed_of(5, 0, 9), "ragged")
    x = wl.materialize(sp).float()
    zero_rows = (x == 0).all(dim=1)
    assert bool(zero_rows[0]) and bool(zero_rows[-1])
    assert 10 <= int(zero_rows.sum()) <= 12                    # row 0, last row, 1% of rows
    live = x[~zero_rows]
    lap = live.abs() > 0.1                                     # mostly Laplace(0, 0.2) draws
    frac = float(lap.float().mean())
    assert 0.05 < frac < 0.1                                   # 10% Laplace, ~61% of them > 0.1
    assert math.isfinite(float(live.abs().max()))


def test_ragged_set():
    shapes = [(s.M, s.N) for s in wl.c5()]
    assert shapes == list(wl.RAGGED_SHAPES)
    assert wl.RAGGED_BLOCKS == ((128, 128), (64, 64), (1, 128))
