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
_FP8 = object()  # placeholder for a weight that is being quantized


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
    pending = []   # (name, tensor) in input order; _FP8 marks a weight in `xs`
    xs = []        # the FP8 weights of the pending group, in order
    nbytes = 0

    def flush():
        nonlocal pending, xs, nbytes
        if not pending:
            return
        items, group = pending, xs
        pending, xs, nbytes = [], [], 0
        outs = iter(quantize_many(group, (bm, bn)) if group else ())
        del group      # the BF16 inputs go once the launch is enqueued
        for name, x in items:
            if x is not _FP8:
                yield name, x
                continue
            q, s = next(outs)
            yield name, q
            yield name + SCALE_SUFFIX, (s.squeeze(-1) if squeeze_scale and s.shape[-1] == 1 else s)

    for name, t in weights:
        if not is_fp8(name, t):
            pending.append((name, t))
            if not xs:
                yield from flush()   # nothing to wait for
            continue
        x = t if (t.dtype is dtype and t.is_contiguous()) else t.to(dtype).contiguous()
        pending.append((name, _FP8))
        xs.append(x)
        nbytes += x.numel() * x.element_size()
        if len(xs) >= group_max or nbytes >= group_bytes:
            yield from flush()
    yield from flush()
