"""The streaming quant_weights loop: ordering, grouping and pass-through on the
CPU with a stand-in for the grouped launch; equality with single calls on
the GPU."""

import pytest
import torch

import fp8_blockwise_weight_amd as fq
from fp8_blockwise_weight_amd import stream


class FakeGroup:
    """Records grouped calls; returns (q, s) markers carrying the input name index."""

    def __init__(self):
        self.calls = []

    def __call__(self, xs, block):
        self.calls.append(len(xs))
        return [(("q", float(x[0, 0])), torch.ones(1, 1) * float(x[0, 0])) for x in xs]


def _weights(n, bias_every=3):
    out = []
    for i in range(n):
        out.append((f"layers.{i}.proj.weight", torch.full((4, 8), float(i), dtype=torch.bfloat16)))
        if i % bias_every == 0:
            out.append((f"layers.{i}.proj.bias", torch.full((8,), float(i))))
    return out


def test_order_names_and_passthrough(monkeypatch):
    fake = FakeGroup()
    monkeypatch.setattr(stream, "quantize_many", fake)
    ws = _weights(7)
    got = list(stream.quant_weights(ws, (128, 128)))
    names = [n for n, _ in got]
    want = []
    for n, _ in ws:
        want += [n, n + "_scale_inv"] if n.endswith("weight") else [n]
    assert names == want
    for n, v in got:
        if n.endswith("bias"):
            assert v.dim() == 1
    # pass-through tensors wait beside the FP8 ones: the 7 weights share one launch
    assert fake.calls == [7]


def test_grouping_limits(monkeypatch):
    fake = FakeGroup()
    monkeypatch.setattr(stream, "quantize_many", fake)
    ws = [(f"w{i}.weight", torch.zeros(4, 8, dtype=torch.bfloat16)) for i in range(10)]
    list(stream.quant_weights(ws, (128, 128), group_max=4))
    assert fake.calls == [4, 4, 2]
    fake.calls.clear()
    list(stream.quant_weights(ws, (128, 128), group_bytes=0))
    assert fake.calls == [1] * 10
    fake.calls.clear()
    list(stream.quant_weights(ws, (128, 128), group_bytes=3 * 64))   # 64 B per tensor
    assert fake.calls == [3, 3, 3, 1]


def test_passthrough_order_with_group_limits(monkeypatch):
    """Group limits cut the queue while pass-through pairs wait in it: every
    pair still comes out in input order, and a leading pass-through is not
    held back."""
    fake = FakeGroup()
    monkeypatch.setattr(stream, "quantize_many", fake)
    ws = [("embed.scale", torch.zeros(3))] + _weights(9, bias_every=2)
    it = stream.quant_weights(ws, (128, 128), group_max=4)
    assert next(it)[0] == "embed.scale"
    assert fake.calls == []
    got = [n for n, _ in it]
    want = []
    for n, _ in ws[1:]:
        want += [n, n + "_scale_inv"] if n.endswith("weight") else [n]
    assert got == want
    assert fake.calls == [4, 4, 1]


def test_missing_block_size_raises(monkeypatch):
    monkeypatch.setattr(stream, "quantize_many", FakeGroup())
    with pytest.raises(ValueError):
        list(stream.quant_weights([("a.weight", torch.zeros(2, 2))], None))


def test_predicate_and_cast(monkeypatch):
    seen = []

    def fake(xs, block):
        seen.extend((x.dtype, x.is_contiguous()) for x in xs)
        return [(x, torch.ones(1, 1)) for x in xs]

    monkeypatch.setattr(stream, "quantize_many", fake)
    ws = [("a.weight", torch.zeros(8, 4).t()), ("b.kv_scale", torch.zeros(1)),
          ("c.weight", torch.zeros(3, 3, dtype=torch.float16))]
    got = list(stream.quant_weights(ws, (128, 128), is_fp8=lambda n, t: n.endswith("weight")))
    assert [n for n, _ in got] == ["a.weight", "a.weight_scale_inv", "b.kv_scale", "c.weight",
                                   "c.weight_scale_inv"]
    assert seen == [(torch.bfloat16, True), (torch.bfloat16, True)]


def test_squeeze_scale(monkeypatch):
    monkeypatch.setattr(stream, "quantize_many",
                        lambda xs, b: [(x, torch.ones(x.shape[0], 1)) for x in xs])
    got = dict(stream.quant_weights([("a.weight", torch.zeros(5, 4))], (1, 128), squeeze_scale=True))
    assert got["a.weight_scale_inv"].shape == (5,)


@pytest.mark.gpu
def test_stream_matches_single_calls(gpu_lib):
    from fp8_blockwise_weight_amd import workloads as wl

    specs = wl.c4_layer(0)[:40] + wl.c2()[:2]
    ws = []
    for sp in specs:
        ws.append((sp.name + ".weight", wl.materialize(sp, "cuda:0")))
        ws.append((sp.name + ".bias", torch.zeros(sp.M, device="cuda:0")))
    out = dict(stream.quant_weights(ws, (128, 128), group_max=16))
    for name, x in ws:
        if name.endswith("bias"):
            assert out[name] is x
            continue
        q, s = fq.quantize(x, (128, 128))
        assert torch.equal(out[name].view(torch.uint8), q.view(torch.uint8)), name
        assert torch.equal(out[name + "_scale_inv"], s), name
