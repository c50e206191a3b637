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

The per-weight host work is what bounds a stream of small matrices (an MoE
layer has hundreds), so each weight's shape, data pointer and device are read
once, here, and the grouped launch takes them as they are (it checks once per
group that the device is a GPU).
"""

from typing import Callable, Iterable, Iterator, Tuple

from . import _quantize_checked, block_shape

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
    first; they must be 2-D and on one GPU.  ``group_bytes=0`` quantizes one
    weight per launch (the pages' one-at-a-time behaviour, lowest peak
    memory).  ``squeeze_scale`` drops a trailing dimension of size 1 from the
    scale, as the SGLang loop does.
    """
    import torch

    bm, bn = block_shape(block_size)  # raises ValueError when the block size is missing
    dtype = dtype or torch.bfloat16
    if dtype is not torch.bfloat16:
        raise TypeError("the quantizer takes BF16 input")
    default = is_fp8 is default_is_fp8
    pending = []   # (name, tensor) in input order; tensor None marks a queued FP8 weight
    shapes = []    # (M, N) of the queued FP8 weights, in order
    ptrs = []      # their data pointers
    xs = []        # the BF16 inputs themselves, alive until their launch is enqueued
    nbytes = 0
    device = None
    index = None

    def flush():
        nonlocal pending, shapes, ptrs, xs, nbytes
        if not pending:
            return
        items, sh, pt = pending, shapes, ptrs
        pending, shapes, ptrs, nbytes = [], [], [], 0
        qs, ss = _quantize_checked(xs, sh, pt, bm, bn, device) if sh else ((), ())
        xs = []        # the BF16 inputs go once the launch is enqueued
        if squeeze_scale:
            ss = [s.squeeze(-1) if s.shape[-1] == 1 else s for s in ss]
        k = 0
        for name, x in items:
            if x is None:
                yield name, qs[k]
                yield name + SCALE_SUFFIX, ss[k]
                k += 1
            else:
                yield name, x

    for name, t in weights:
        if not ((name.endswith("weight") and t.ndim == 2) if default else is_fp8(name, t)):
            pending.append((name, t))
            if not shapes:
                yield from flush()   # nothing to wait for
            continue
        if not (t.dtype is dtype and t.is_contiguous()):
            t = t.to(dtype).contiguous()
        d = t.get_device()           # -1 off the GPU; the grouped call refuses that device
        if d != index:
            if index is not None:
                raise ValueError(f"{name}: FP8 weights must all be on one GPU ({t.device}, {device})")
            index, device = d, t.device
        try:
            M, N = t.shape
        except ValueError:
            raise TypeError(f"{name}: FP8 weights must be 2-D, got shape {tuple(t.shape)}") from None
        pending.append((name, None))
        shapes.append((M, N))
        ptrs.append(t.data_ptr())
        xs.append(t)
        nbytes += 2 * M * N
        if nbytes >= group_bytes or len(shapes) >= group_max:
            yield from flush()
    yield from flush()
