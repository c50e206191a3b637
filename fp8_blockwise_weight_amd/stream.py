"""Streaming FP8 quantization of a (name, tensor) weight stream.

The page "vllm_fp8_utils.py" (section 3, ``quant_weights``) describes the
loop the rollout stack runs on every weight sync: walk the (name, tensor)
pairs, pass non-FP8 weights through unchanged, and for each FP8 weight yield
the quantized tensor under its own name followed by its descale under
``<name>_scale_inv``, releasing memory as it goes.  The SGLang variant in
"[rollout, sglang] feat: support blockwise fp8 rollout" (review excerpt)
raises when no block size is configured and squeezes a trailing singleton
off the scale.

Here FP8 weights are batched into one grouped launch (``quantize_many``),
bounded by ``group_bytes`` of BF16 input and ``group_max`` tensors, so
thousands of small expert matrices cost a handful of launches.  Pass-through
pairs (norms, biases) wait in the queue beside them instead of cutting the
group, so a decoder layer's projections share a launch.  Output order is
the input order.  Which weights are FP8 is a caller predicate (the pages ask
the inference engine's module types; this library has no engine, so the
default is "a 2-D tensor whose name ends in ``weight``").
"""

from typing import Callable, Iterable, Iterator, Tuple

from . import block_shape, quantize_many

SCALE_SUFFIX = "_scale_inv"


def default_is_fp8(name: str, tensor) -> bool:
    """2-D tensors named ``...weight`` (linear and expert weights)."""
    return name.endswith("weight") and tensor.dim() == 2


def quant_weights(weights: Iterable[Tuple[str, object]], block_size=(128, 128),
                  is_fp8: Callable[[str, object], bool] = default_is_fp8, dtype=None,
                  group_bytes: int = 1 << 30, group_max: int = 512,
                  squeeze_scale: bool = False) -> Iterator[Tuple[str, object]]:
    """Yield ``(name, tensor)`` pairs with every FP8 weight quantized.

    For an FP8 weight ``k`` the stream carries ``(k, q)`` and then
    ``(k + "_scale_inv", scale_inv)``; other pairs pass through unchanged.
    Weights are cast to ``dtype`` (default bfloat16) and made contiguous
    first.  ``group_bytes=0`` quantizes one weight per launch (the pages'
    one-at-a-time behaviour, lowest peak memory).  ``squeeze_scale`` drops
    a trailing dimension of size 1 from the scale, as the SGLang loop does.
    """
    import torch

    bm, bn = block_shape(block_size)  # raises ValueError when the block size is missing
    dtype = dtype or torch.bfloat16
    pending = []     # (name, tensor, quantize?) in input order
    state = {"bytes": 0, "count": 0}

    def flush():
        if not pending:
            return
        items = list(pending)
        pending.clear()
        state["bytes"] = state["count"] = 0
        xs = [x for _, x, fp8 in items if fp8]
        outs = iter(quantize_many(xs, (bm, bn)) if xs else [])
        del xs
        items = [(name, None if fp8 else x, fp8) for name, x, fp8 in items]  # drop BF16 inputs
        for name, x, fp8 in items:
            if not fp8:
                yield name, x
                continue
            q, s = next(outs)
            yield name, q
            yield name + SCALE_SUFFIX, (s.squeeze(-1) if squeeze_scale and s.shape[-1] == 1 else s)

    for name, t in weights:
        if not is_fp8(name, t):
            pending.append((name, t, False))
            if not state["count"]:
                yield from flush()   # nothing to wait for
            continue
        x = t if (t.dtype == dtype and t.is_contiguous()) else t.to(dtype).contiguous()
        pending.append((name, x, True))
        state["count"] += 1
        state["bytes"] += x.numel() * x.element_size()
        if state["count"] >= group_max or state["bytes"] >= group_bytes:
            yield from flush()
    yield from flush()
