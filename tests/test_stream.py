"""The streaming quant_weights loop: ordering, grouping and pass-through on the
CPU with a stand-in for the grouped launch; on the GPU every yielded code
and descale against the oracle, with the order, the pass-through pairs, the
casts and the squeezed descale checked too."""

import pytest
import torch

import fp8_blockwise_weight_amd as fq
from fp8_blockwise_weight_amd import stream


class FakeGroup:
    """Stands in for the grouped launch: records the group sizes, returns
    marker outputs (the input's first value as q, a 1x1 scale)."""

    def __init__(self):
        self.calls = []

    def __call__(self, xs, shapes, ptrs, bm, bn, dev):
        assert [tuple(x.shape) for x in xs] == list(shapes)
        assert [x.data_ptr() for x in xs] == list(ptrs)
        self.calls.append(len(xs))
        return ([("q", float(x[0, 0])) for x in xs], [torch.ones(1, 1) * float(x[0, 0]) for x in xs])


def _weights(n, bias_every=3):
    out = []
    for i in range(n):
        out.append((f"layers.{i}.proj.weight", torch.full((4, 8), float(i), dtype=torch.bfloat16)))
        if i % bias_every == 0:
            out.append((f"layers.{i}.proj.bias", torch.full((8,), float(i))))
    return out


def test_order_names_and_passthrough(monkeypatch):
    fake = FakeGroup()
    monkeypatch.setattr(stream, "_quantize_checked", fake)
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
    monkeypatch.setattr(stream, "_quantize_checked", fake)
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
    monkeypatch.setattr(stream, "_quantize_checked", fake)
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
    monkeypatch.setattr(stream, "_quantize_checked", FakeGroup())
    with pytest.raises(ValueError):
        list(stream.quant_weights([("a.weight", torch.zeros(2, 2))], None))


def test_predicate_and_cast(monkeypatch):
    seen = []

    def fake(xs, shapes, ptrs, bm, bn, dev):
        seen.extend((x.dtype, x.is_contiguous()) for x in xs)
        return list(xs), [torch.ones(1, 1) for _ in xs]

    monkeypatch.setattr(stream, "_quantize_checked", fake)
    ws = [("a.weight", torch.zeros(8, 4).t()), ("b.kv_scale", torch.zeros(1)),
          ("c.weight", torch.zeros(3, 3, dtype=torch.float16))]
    got = list(stream.quant_weights(ws, (128, 128), is_fp8=lambda n, t: n.endswith("weight")))
    assert [n for n, _ in got] == ["a.weight", "a.weight_scale_inv", "b.kv_scale", "c.weight",
                                   "c.weight_scale_inv"]
    assert seen == [(torch.bfloat16, True), (torch.bfloat16, True)]


def test_weights_must_be_2d(monkeypatch):
    monkeypatch.setattr(stream, "_quantize_checked", FakeGroup())
    with pytest.raises(TypeError, match="2-D"):
        list(stream.quant_weights([("a.weight", torch.zeros(2, 2, 2))], (128, 128),
                                  is_fp8=lambda n, t: True))


def test_cpu_weights_are_refused():
    """Without the stand-in: the grouped call refuses a group off the GPU
    before anything reaches the library."""
    with pytest.raises(TypeError, match="on a GPU"):
        list(stream.quant_weights([("a.weight", torch.zeros(4, 8, dtype=torch.bfloat16))], (128, 128)))


def test_squeeze_scale(monkeypatch):
    monkeypatch.setattr(stream, "_quantize_checked",
                        lambda xs, sh, p, bm, bn, d: (list(xs), [torch.ones(x.shape[0], 1) for x in xs]))
    got = dict(stream.quant_weights([("a.weight", torch.zeros(5, 4))], (1, 128), squeeze_scale=True))
    assert got["a.weight_scale_inv"].shape == (5,)


def _stream_inputs(dev):
    """A dense decoder layer and a slice of an MoE layer in model order, with
    norms (1-D, passed through), a bias and an fp16 weight (cast to BF16)."""
    from fp8_blockwise_weight_amd import workloads as wl

    ws = []
    for sp in wl.c2():
        if sp.name.endswith("q_proj"):
            ws.append(("layers.0.input_layernorm.weight", torch.ones(4096, dtype=torch.bfloat16, device=dev)))
        if sp.name.endswith("gate_proj"):
            ws.append(("layers.0.post_attention_layernorm.weight",
                       torch.ones(4096, dtype=torch.bfloat16, device=dev)))
        ws.append((sp.name + ".weight", wl.materialize(sp, dev)))
    ws.append(("layers.0.o_proj.bias", torch.zeros(4096, device=dev)))
    for sp in wl.c4_layer(1)[:96]:
        ws.append((sp.name + ".weight", wl.materialize(sp, dev)))
    half = (torch.randn((640, 384), generator=torch.Generator(device=dev).manual_seed(7), device=dev)
            * 0.05).to(torch.float16)
    ws.append(("lm_head.weight", half))
    return ws


@pytest.mark.gpu
@pytest.mark.parametrize("limits", [dict(group_max=16, group_bytes=300 << 20),
                                    dict(group_max=512, group_bytes=1 << 30),
                                    dict(group_bytes=0)])
def test_stream_matches_oracle(gpu_lib, oracle_pool, limits):
    """Every yielded (name, q) and (name + "_scale_inv", s) pair against the
    oracle, byte for byte and bit for bit, with groups cut inside the dense
    layer and inside the MoE slice (or one tensor per launch); pass-through
    pairs come out as the same objects, and the order is the input order."""
    from gpu_helpers import FullOracleCheck

    dev = "cuda:0"
    ws = _stream_inputs(dev)
    out = list(stream.quant_weights(ws, (128, 128), **limits))
    want = []
    for n, t in ws:
        want += [n, n + "_scale_inv"] if (n.endswith("weight") and t.dim() == 2) else [n]
    assert [n for n, _ in out] == want
    got = dict(out)
    chk = FullOracleCheck(oracle_pool, 128, 128, f"stream {limits}")
    for name, t in ws:
        if not (name.endswith("weight") and t.dim() == 2):
            assert got[name] is t, name
            continue
        q, s = got[name], got[name + "_scale_inv"]
        assert q.dtype == torch.float8_e4m3fn and s.dtype == torch.float32, name
        assert tuple(q.shape) == tuple(t.shape) and tuple(s.shape) == fq.scale_shape(*t.shape, 128, 128)
        chk.add(name, t.to(torch.bfloat16), q, s)
    n, values = chk.finish()
    assert n == 7 + 96 + 1
    del out, got


@pytest.mark.gpu
def test_stream_squeezed_scale_matches_oracle(gpu_lib):
    """[1,128] blocks on 128-wide weights give an [M, 1] descale; with
    ``squeeze_scale`` it comes out as [M] and still equals the oracle's."""
    from gpu_helpers import assert_matches_oracle

    g = torch.Generator(device="cuda:0").manual_seed(11)
    ws = [(f"e{i}.weight", (torch.randn((m, 128), generator=g, device="cuda:0") * 0.03).to(torch.bfloat16))
          for i, m in enumerate((1, 77, 300))]
    got = dict(stream.quant_weights(ws, (1, 128), squeeze_scale=True))
    for name, x in ws:
        s = got[name + "_scale_inv"]
        assert tuple(s.shape) == (x.shape[0],), name
        assert_matches_oracle(x, got[name], s.unsqueeze(-1), 1, 128, name)
