"""Python binding of libfp8bq (blockwise FP8 e4m3fn weight quantization, gfx950).

Argument marshalling only: every step of the quantization runs in the HIP
kernels of ``libfp8bq.so``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or the device is
not a gfx950, the calls raise.

The entry point mirrors ``scaled_fp8_blockwise(data_hp, weight_block_size)``
of the page "fp8_kernel.py — FP8 量化内核" (section 1): an [M, N] matrix
and a [BLOCK_M, BLOCK_N] block size in, ``(fp8_data, descale)`` out, with the
descale shaped [ceil(M/bm), ceil(N/bn)].  ``quantize_many`` is the grouped
form of the per-weight loop of the page "vllm_fp8_utils.py" (section 3).
"""

import ctypes
import os
import struct
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8bq.so")

# Status codes of include/fp8bq.h
OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED_DEVICE = 2
ERR_WORKSPACE = 3
ERR_HIP = 4

E4M3_MAX = 448.0
EPS = 1e-10
NOALLOC_MAX_TENSORS = 16384   # FP8BQ_NOALLOC_MAX_TENSORS

# Every symbol include/fp8bq.h declares.
EXPORTS = (
    "fp8bq_quantize",
    "fp8bq_many_workspace_bytes",
    "fp8bq_quantize_many",
    "fp8bq_quantize_many_noalloc",
    "fp8bq_encode_e4m3",
    "fp8bq_dequantize",
    "fp8bq_dequantize_many",
    "fp8bq_tile_amax",
    "fp8bq_quantize_amax",
    "fp8bq_tile_amax_many",
    "fp8bq_quantize_amax_many",
    "fp8bq_row_shard_edges",
    "fp8bq_row_shards_begin",
    "fp8bq_row_shards_finish",
    "fp8bq_set_resident_wait_us",
    "fp8bq_status_string",
    "fp8bq_last_hip_error",
)


class DqEntry(ctypes.Structure):
    """``fp8bq_dq_tensor`` of include/fp8bq.h (40 bytes, no padding)."""
    _fields_ = [("q", ctypes.c_void_p), ("scale_inv", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64)]


class TensorEntry(ctypes.Structure):
    """``fp8bq_tensor`` of include/fp8bq.h (40 bytes, no padding)."""

    _fields_ = [
        ("x", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("scale_inv", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
    ]


class Fp8bqError(RuntimeError):
    def __init__(self, where: str, status: int, hip_error: int):
        self.status = status
        self.hip_error = hip_error
        text = load_library().fp8bq_status_string(status).decode()
        super().__init__(f"{where}: {text} (status {status}, hip error {hip_error})")


class ShardEntry(ctypes.Structure):
    """``fp8bq_shard`` of include/fp8bq.h (56 bytes, no padding)."""

    _fields_ = [
        ("x", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("amax", ctypes.c_void_p),
        ("scale_inv", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("row_phase", ctypes.c_int32),
        ("col_phase", ctypes.c_int32),
    ]


class RowShardEntry(ctypes.Structure):
    """``fp8bq_row_shard`` of include/fp8bq.h (64 bytes, no padding)."""

    _fields_ = [
        ("x", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("scale_inv", ctypes.c_void_p),
        ("top_amax", ctypes.c_void_p),
        ("bottom_amax", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("row_phase", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libfp8bq.so (built in-tree by ``fp8_blockwise_weight_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_blockwise_weight_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.fp8bq_quantize.argtypes = [c_vp, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp]
    lib.fp8bq_quantize.restype = ctypes.c_int
    lib.fp8bq_many_workspace_bytes.argtypes = [c_i32]
    lib.fp8bq_many_workspace_bytes.restype = ctypes.c_size_t
    lib.fp8bq_quantize_many.argtypes = [ctypes.POINTER(TensorEntry), c_i32, c_i32, c_i32, c_vp,
                                        ctypes.c_size_t, c_vp]
    lib.fp8bq_quantize_many.restype = ctypes.c_int
    lib.fp8bq_quantize_many_noalloc.argtypes = [ctypes.POINTER(TensorEntry), c_i32, c_i32, c_i32, c_vp]
    lib.fp8bq_quantize_many_noalloc.restype = ctypes.c_int
    lib.fp8bq_dequantize.argtypes = [c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_vp, c_i32, c_vp]
    lib.fp8bq_dequantize.restype = ctypes.c_int
    lib.fp8bq_dequantize_many.argtypes = [ctypes.POINTER(DqEntry), c_i32, c_i32, c_i32, c_i32, c_vp]
    lib.fp8bq_dequantize_many.restype = ctypes.c_int
    lib.fp8bq_tile_amax.argtypes = [c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.fp8bq_tile_amax.restype = ctypes.c_int
    lib.fp8bq_quantize_amax.argtypes = [c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_vp,
                                        c_vp, c_vp, c_vp]
    lib.fp8bq_quantize_amax.restype = ctypes.c_int
    for name in ("fp8bq_tile_amax_many", "fp8bq_quantize_amax_many"):
        getattr(lib, name).argtypes = [ctypes.POINTER(ShardEntry), c_i32, c_i32, c_i32, c_vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.fp8bq_row_shard_edges.argtypes = [c_i64, c_i32, c_i32, ctypes.POINTER(c_i64),
                                          ctypes.POINTER(c_i64)]
    lib.fp8bq_row_shard_edges.restype = ctypes.c_int
    lib.fp8bq_row_shards_begin.argtypes = [ctypes.POINTER(RowShardEntry), c_i32, c_i32, c_i32, c_vp,
                                           ctypes.c_size_t, c_vp, c_vp]
    lib.fp8bq_row_shards_begin.restype = ctypes.c_int
    lib.fp8bq_row_shards_finish.argtypes = [ctypes.POINTER(RowShardEntry), c_i32, c_i32, c_i32, c_vp]
    lib.fp8bq_row_shards_finish.restype = ctypes.c_int
    lib.fp8bq_encode_e4m3.argtypes = [c_vp, c_vp, c_i64, c_vp]
    lib.fp8bq_encode_e4m3.restype = ctypes.c_int
    lib.fp8bq_set_resident_wait_us.argtypes = [c_i64]
    lib.fp8bq_set_resident_wait_us.restype = ctypes.c_int
    lib.fp8bq_status_string.argtypes = [ctypes.c_int]
    lib.fp8bq_status_string.restype = ctypes.c_char_p
    lib.fp8bq_last_hip_error.argtypes = []
    lib.fp8bq_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(where: str, status: int) -> None:
    if status != OK:
        raise Fp8bqError(where, status, load_library().fp8bq_last_hip_error())


def block_shape(block_size) -> Tuple[int, int]:
    """Validate a block size: the SGLang loop raises when it is missing."""
    if block_size is None:
        raise ValueError("weight_block_size is required (got None)")
    bm, bn = (int(v) for v in block_size)
    if bm < 1 or bn < 1:
        raise ValueError(f"block size must be positive, got {tuple(block_size)}")
    return bm, bn


def scale_shape(M: int, N: int, bm: int, bn: int) -> Tuple[int, int]:
    return (-(-M // bm), -(-N // bn))


def _check_input(x) -> None:
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D torch.bfloat16 tensor")
    if not x.is_cuda:
        raise TypeError("x must be on a GPU (there is no CPU implementation)")
    if not x.is_contiguous():
        raise TypeError("x must be contiguous row-major")


def _check_buffer(t, shape, elem_size: int, device, what: str) -> None:
    """A caller-supplied output must match exactly: the kernels write every
    byte of it, and nothing outside it."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.element_size() != elem_size:
        raise TypeError(f"{what} must have {elem_size}-byte elements, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")


def _check_outputs(out, M: int, N: int, bm: int, bn: int, device) -> None:
    import torch

    q, s = out
    _check_buffer(q, (M, N), 1, device, "q")
    _check_buffer(s, scale_shape(M, N, bm, bn), 4, device, "scale_inv")
    if s.dtype != torch.float32:
        raise TypeError("scale_inv must be float32")


def _stream(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def quantize(x, block_size=(128, 128), out=None):
    """Quantize one BF16 [M, N] GPU tensor.

    Returns ``(q, scale_inv)``: ``q`` is torch.float8_e4m3fn [M, N] and
    ``scale_inv`` float32 [ceil(M/bm), ceil(N/bn)]; dequantize with
    ``q.float() * scale_inv`` expanded over each block.  ``out`` may supply
    preallocated ``(q, scale_inv)``.  Work is enqueued on the current stream.
    """
    import torch

    bm, bn = block_shape(block_size)
    _check_input(x)
    M, N = x.shape
    if out is None:
        q = torch.empty((M, N), dtype=torch.float8_e4m3fn, device=x.device)
        s = torch.empty(scale_shape(M, N, bm, bn), dtype=torch.float32, device=x.device)
    else:
        _check_outputs(out, M, N, bm, bn, x.device)
        q, s = out
    lib = load_library()
    with torch.cuda.device(x.device):
        _check("fp8bq_quantize",
               lib.fp8bq_quantize(x.data_ptr(), M, N, bm, bn, q.data_ptr(), s.data_ptr(),
                                  _stream(x.device)))
    return q, s


def workspace_bytes(count: int) -> int:
    return int(load_library().fp8bq_many_workspace_bytes(int(count)))


_ENTRY = struct.Struct("=QQQqq")  # fp8bq_tensor: x, q, scale_inv, M, N


def make_entries(tensors: Sequence, outputs: Sequence) -> ctypes.Array:
    """The host ``fp8bq_tensor`` array of a grouped call."""
    buf = bytearray(_ENTRY.size * len(tensors))
    off = 0
    for x, (q, s) in zip(tensors, outputs):
        M, N = x.shape
        _ENTRY.pack_into(buf, off, x.data_ptr(), q.data_ptr(), s.data_ptr(), M, N)
        off += _ENTRY.size
    return (TensorEntry * len(tensors)).from_buffer(buf)


def _plan_outputs(shapes: Sequence, ptrs: Sequence, bm: int, bn: int, device):
    """Outputs for a grouped call: one q buffer and one scale buffer per
    distinct row length N, holding the tensors' [M, N] / [TM, TN] outputs
    one after another in input order (contiguous and disjoint).  Two
    allocations per row length instead of two per tensor: for lists of
    thousands of small matrices the allocations, not the kernel, set the
    pace.  ``shapes`` and ``ptrs`` are the inputs' (M, N) and data pointers.
    Returns the ``fp8bq_tensor`` array (a bytearray) filled from the buffers'
    addresses, and a function that cuts the per-tensor views as two lists
    (q views, scale views) in input order; calling it after the launch lets
    the device start while the host builds them."""
    import torch

    n = len(shapes)
    by_n = {}
    for i, (M, N) in enumerate(shapes):
        g = by_n.get(N)
        if g is None:
            by_n[N] = g = ([], [])
        g[0].append(i)
        g[1].append(M)
    entries = bytearray(_ENTRY.size * n)
    pack, size = _ENTRY.pack_into, _ENTRY.size
    plan = []
    for N, (idx, ms) in by_n.items():
        tms = [-(-m // bm) for m in ms]
        TN = -(-N // bn)
        qbuf = torch.empty((sum(ms), N), dtype=torch.float8_e4m3fn, device=device)
        sbuf = torch.empty((sum(tms), TN), dtype=torch.float32, device=device)
        qp, sp = qbuf.data_ptr(), sbuf.data_ptr()
        for i, m, tm in zip(idx, ms, tms):
            pack(entries, size * i, ptrs[i], qp, sp, m, N)
            qp += m * N
            sp += 4 * tm * TN
        plan.append((idx, qbuf, sbuf, ms, tms))

    def views():
        # outputs never require grad: views without autograd's view tracking
        split = torch.unsafe_split_with_sizes
        if len(plan) == 1:                 # one row length: the splits are in input order
            _, qbuf, sbuf, ms, tms = plan[0]
            return list(split(qbuf, ms)), list(split(sbuf, tms))
        qs, ss = [None] * n, [None] * n
        for idx, qbuf, sbuf, ms, tms in plan:
            for i, q, sc in zip(idx, split(qbuf, ms), split(sbuf, tms)):
                qs[i] = q
                ss[i] = sc
        return qs, ss

    return entries, views


def _launch_many(arr, n: int, bm: int, bn: int, dev, workspace=None) -> None:
    """fp8bq_quantize_many on ``dev``'s current stream (a workspace is made
    when the table does not fit the kernel arguments and none is given)."""
    import torch

    lib = load_library()
    need = int(lib.fp8bq_many_workspace_bytes(n))
    if workspace is None:
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the tensors' device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        _check("fp8bq_quantize_many",
               lib.fp8bq_quantize_many(arr, n, bm, bn, ws_ptr, ws_bytes, _stream(dev)))


def _quantize_checked(xs: Sequence, shapes: Sequence, ptrs: Sequence, bm: int, bn: int, dev):
    """One grouped call over inputs already checked (BF16, 2-D, contiguous,
    all on ``dev``), given with their shapes and data pointers.  Returns the
    q views and the scale views, two lists in input order."""
    if dev.type != "cuda":
        raise TypeError("x must be on a GPU (there is no CPU implementation)")
    entries, views = _plan_outputs(shapes, ptrs, bm, bn, dev)
    n = len(shapes)
    _launch_many((TensorEntry * n).from_buffer(entries), n, bm, bn, dev)
    return views()


def quantize_many(tensors: Sequence, block_size=(128, 128), outputs: Optional[Sequence] = None,
                  workspace=None) -> List:
    """Quantize a list of BF16 GPU tensors (same device, one block size) in one launch.

    Returns a list of ``(q, scale_inv)`` pairs in input order.  Outputs the
    call allocates are row views into one buffer per distinct N (a view
    keeps its buffer alive).  ``outputs`` and ``workspace`` (a uint8 GPU
    tensor of at least ``workspace_bytes``) may be preallocated.
    """
    import torch

    bm, bn = block_shape(block_size)
    tensors = list(tensors)
    if not tensors:
        return []
    dev = tensors[0].device
    index = tensors[0].get_device()
    bf16 = torch.bfloat16
    shapes, ptrs = [], []
    for x in tensors:
        # the common case in one expression; _check_input names what is wrong
        if not (isinstance(x, torch.Tensor) and x.dtype is bf16 and x.dim() == 2 and x.is_cuda
                and x.is_contiguous()):
            _check_input(x)
        if x.get_device() != index:
            raise ValueError("all tensors of one grouped call must be on the same device")
        shapes.append(tuple(x.shape))
        ptrs.append(x.data_ptr())
    n = len(tensors)
    if outputs is None:
        entries, views = _plan_outputs(shapes, ptrs, bm, bn, dev)
        _launch_many((TensorEntry * n).from_buffer(entries), n, bm, bn, dev, workspace)
        return list(zip(*views()))
    outputs = list(outputs)
    if len(outputs) != n:
        raise ValueError("outputs must hold one (q, scale_inv) pair per tensor")
    for (M, N), out in zip(shapes, outputs):
        _check_outputs(out, M, N, bm, bn, dev)
    _launch_many(make_entries(tensors, outputs), n, bm, bn, dev, workspace)
    return outputs


def quantize_many_noalloc(tensors: Sequence, outputs: Sequence, block_size=(128, 128)) -> List:
    """``quantize_many`` into caller-supplied outputs through
    ``fp8bq_quantize_many_noalloc``: no device memory is allocated anywhere in
    the call (lists beyond 512 tensors use the library's per-device table
    block).  Calls that overlap on one GPU race on that block; order them on
    one stream.  Returns ``outputs``."""
    import torch

    bm, bn = block_shape(block_size)
    tensors, outputs = list(tensors), list(outputs)
    if len(outputs) != len(tensors):
        raise ValueError("outputs must hold one (q, scale_inv) pair per tensor")
    if not tensors:
        return outputs
    if len(tensors) > NOALLOC_MAX_TENSORS:
        raise ValueError(f"at most {NOALLOC_MAX_TENSORS} tensors per call, got {len(tensors)}")
    dev = tensors[0].device
    for x, out in zip(tensors, outputs):
        _check_input(x)
        if x.device != dev:
            raise ValueError("all tensors of one grouped call must be on the same device")
        _check_outputs(out, *x.shape, bm, bn, dev)
    arr = make_entries(tensors, outputs)
    with torch.cuda.device(dev):
        _check("fp8bq_quantize_many_noalloc",
               load_library().fp8bq_quantize_many_noalloc(arr, len(tensors), bm, bn, _stream(dev)))
    return outputs


def dequantize(q, scale_inv, block_size=(128, 128), out_dtype=None, out=None):
    """x_hat = decode(q) * scale_inv (per block), as float32 or bfloat16 [M, N].

    ``q`` is a float8_e4m3fn (or uint8) GPU tensor [M, N]; ``scale_inv`` the
    float32 [ceil(M/bm), ceil(N/bn)] descale from ``quantize``.
    """
    import torch

    bm, bn = block_shape(block_size)
    out_dtype = out_dtype or torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if q.dim() != 2 or q.element_size() != 1 or not q.is_cuda or not q.is_contiguous():
        raise TypeError("q must be a contiguous 2-D one-byte GPU tensor")
    M, N = q.shape
    if tuple(scale_inv.shape) != scale_shape(M, N, bm, bn) or scale_inv.dtype != torch.float32 \
            or not scale_inv.is_contiguous():
        raise TypeError("scale_inv must be contiguous float32 [ceil(M/bm), ceil(N/bn)]")
    if scale_inv.device != q.device:
        raise ValueError("scale_inv must be on q's device")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=q.device)
    else:
        _check_buffer(out, (M, N), 4 if out_dtype == torch.float32 else 2, q.device, "out")
        if out.dtype != out_dtype:
            raise TypeError(f"out must be {out_dtype}")
    code = 0 if out_dtype == torch.float32 else 1
    with torch.cuda.device(q.device):
        _check("fp8bq_dequantize",
               load_library().fp8bq_dequantize(q.data_ptr(), scale_inv.data_ptr(), M, N, bm, bn,
                                               out.data_ptr(), code, _stream(q.device)))
    return out


def dequantize_many(qs: Sequence, scales: Sequence, block_size=(128, 128), out_dtype=None,
                    outs: Optional[Sequence] = None) -> List:
    """``dequantize`` over a list of (q, scale_inv) pairs with one block size
    and one output type, in grouped launches (``fp8bq_dequantize_many``)."""
    import torch

    bm, bn = block_shape(block_size)
    out_dtype = out_dtype or torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if len(qs) != len(scales) or (outs is not None and len(outs) != len(qs)):
        raise ValueError("qs, scales (and outs) must have the same length")
    if not qs:
        return []
    device = qs[0].device
    esize = 4 if out_dtype == torch.float32 else 2
    table = (DqEntry * len(qs))()
    result = []
    for i, (q, s) in enumerate(zip(qs, scales)):
        if q.dim() != 2 or q.element_size() != 1 or not q.is_cuda or not q.is_contiguous():
            raise TypeError(f"qs[{i}] must be a contiguous 2-D one-byte GPU tensor")
        if q.device != device:
            raise ValueError("every tensor must be on one device")
        M, N = q.shape
        if tuple(s.shape) != scale_shape(M, N, bm, bn) or s.dtype != torch.float32 \
                or not s.is_contiguous() or s.device != device:
            raise TypeError(f"scales[{i}] must be contiguous float32 [ceil(M/bm), ceil(N/bn)] on q's device")
        if outs is None:
            o = torch.empty((M, N), dtype=out_dtype, device=device)
        else:
            o = outs[i]
            _check_buffer(o, (M, N), esize, device, f"outs[{i}]")
            if o.dtype != out_dtype:
                raise TypeError(f"outs[{i}] must be {out_dtype}")
        table[i] = DqEntry(q.data_ptr(), s.data_ptr(), o.data_ptr(), M, N)
        result.append(o)
    code = 0 if out_dtype == torch.float32 else 1
    with torch.cuda.device(device):
        _check("fp8bq_dequantize_many",
               load_library().fp8bq_dequantize_many(table, len(qs), bm, bn, code, _stream(device)))
    return result


def local_grid(M: int, N: int, bm: int, bn: int, phase=(0, 0)) -> Tuple[int, int]:
    """Tile grid of a shard whose element (0,0) sits at ``phase`` inside a tile."""
    rp, cp = phase
    if not (0 <= rp < bm and 0 <= cp < bn):
        raise ValueError("phase must satisfy 0 <= phase < block")
    return (-(-(rp + M) // bm), -(-(cp + N) // bn))


def tile_amax(x, block_size=(128, 128), phase=(0, 0), out=None):
    """Per-tile max |x| (float32 [TMl, TNl]) of a BF16 shard at tile ``phase``.

    Combine the results of shards that share tiles with an element-wise max
    (exact), then pass the full maxima to ``quantize_with_amax``.
    """
    import torch

    bm, bn = block_shape(block_size)
    _check_input(x)
    M, N = x.shape
    shape = local_grid(M, N, bm, bn, phase)
    if out is not None:
        _check_buffer(out, shape, 4, x.device, "amax")
        if out.dtype != torch.float32:
            raise TypeError("amax must be float32")
    amax = out if out is not None else torch.empty(shape, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check("fp8bq_tile_amax",
               load_library().fp8bq_tile_amax(x.data_ptr(), M, N, bm, bn, phase[0], phase[1],
                                              amax.data_ptr(), _stream(x.device)))
    return amax


def quantize_with_amax(x, amax, block_size=(128, 128), phase=(0, 0), out=None):
    """Quantize a BF16 shard with given whole-tile maxima ``amax`` [TMl, TNl].

    Returns ``(q, scale_inv)``; ``scale_inv`` covers the shard's tiles.
    """
    import torch

    bm, bn = block_shape(block_size)
    _check_input(x)
    M, N = x.shape
    shape = local_grid(M, N, bm, bn, phase)
    _check_buffer(amax, shape, 4, x.device, "amax")
    if amax.dtype != torch.float32:
        raise TypeError("amax must be float32")
    if out is None:
        q = torch.empty((M, N), dtype=torch.float8_e4m3fn, device=x.device)
        s = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        q, s = out
        _check_buffer(q, (M, N), 1, x.device, "q")
        _check_buffer(s, shape, 4, x.device, "scale_inv")
        if s.dtype != torch.float32:
            raise TypeError("scale_inv must be float32")
    with torch.cuda.device(x.device):
        _check("fp8bq_quantize_amax",
               load_library().fp8bq_quantize_amax(x.data_ptr(), M, N, bm, bn, phase[0], phase[1],
                                                  amax.data_ptr(), q.data_ptr(), s.data_ptr(),
                                                  _stream(x.device)))
    return q, s


def _shard_table(xs, phases, qs, amaxs, scales) -> ctypes.Array:
    arr = (ShardEntry * len(xs))()
    for e, x, ph, q, a, s in zip(arr, xs, phases, qs, amaxs, scales):
        e.x, e.amax = x.data_ptr(), a.data_ptr()
        e.q = q.data_ptr() if q is not None else None
        e.scale_inv = s.data_ptr() if s is not None else None
        e.M, e.N = x.shape
        e.row_phase, e.col_phase = ph
    return arr


def _shard_inputs(xs, block_size, phases):
    bm, bn = block_shape(block_size)
    xs = list(xs)
    phases = [tuple(int(v) for v in p) for p in (phases if phases is not None else [(0, 0)] * len(xs))]
    if len(phases) != len(xs):
        raise ValueError("phases must hold one (row_phase, col_phase) per shard")
    dev = xs[0].device if xs else None
    for x in xs:
        _check_input(x)
        if x.device != dev:
            raise ValueError("all shards of one grouped call must be on the same device")
    grids = [local_grid(*x.shape, bm, bn, p) for x, p in zip(xs, phases)]
    return bm, bn, xs, phases, dev, grids


def tile_amax_many(xs: Sequence, block_size=(128, 128), phases=None) -> List:
    """``tile_amax`` of every shard of a list (one block size), in grouped launches."""
    import torch

    bm, bn, xs, phases, dev, grids = _shard_inputs(xs, block_size, phases)
    if not xs:
        return []
    amaxs = [torch.empty(g, dtype=torch.float32, device=dev) for g in grids]
    arr = _shard_table(xs, phases, [None] * len(xs), amaxs, [None] * len(xs))
    with torch.cuda.device(dev):
        _check("fp8bq_tile_amax_many",
               load_library().fp8bq_tile_amax_many(arr, len(xs), bm, bn, _stream(dev)))
    return amaxs


def quantize_with_amax_many(xs: Sequence, amaxs: Sequence, block_size=(128, 128),
                            phases=None) -> List:
    """``quantize_with_amax`` of every shard of a list, in grouped launches.
    Returns ``(q, scale_inv)`` pairs in input order."""
    import torch

    bm, bn, xs, phases, dev, grids = _shard_inputs(xs, block_size, phases)
    amaxs = list(amaxs)
    if len(amaxs) != len(xs):
        raise ValueError("amaxs must hold one maxima tensor per shard")
    if not xs:
        return []
    for a, g in zip(amaxs, grids):
        _check_buffer(a, g, 4, dev, "amax")
        if a.dtype != torch.float32:
            raise TypeError("amax must be float32")
    qs = [torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev) for x in xs]
    scales = [torch.empty(g, dtype=torch.float32, device=dev) for g in grids]
    arr = _shard_table(xs, phases, qs, amaxs, scales)
    with torch.cuda.device(dev):
        _check("fp8bq_quantize_amax_many",
               load_library().fp8bq_quantize_amax_many(arr, len(xs), bm, bn, _stream(dev)))
    return list(zip(qs, scales))


def row_shard_edges(M: int, bm: int, row_phase: int) -> Tuple[int, int]:
    """(top, bottom): how many of a row shard's first and last rows lie in
    tile rows that shards above and below may hold too
    (``fp8bq_row_shard_edges``); the rows between are whole tile rows."""
    top, bottom = ctypes.c_int64(), ctypes.c_int64()
    _check("fp8bq_row_shard_edges",
           load_library().fp8bq_row_shard_edges(int(M), int(bm), int(row_phase), ctypes.byref(top),
                                                ctypes.byref(bottom)))
    return top.value, bottom.value


class RowShards:
    """One quantize-before-gather of row shards in flight, between
    ``row_shards_begin`` and ``row_shards_finish``.

    ``outputs`` holds (q, scale_inv) per shard.  ``edges`` holds, per shard,
    (top, bottom): the fp32 [TN] maxima of the tile rows its first and last
    rows share with other shards, or None where it has no such rows.  They
    are the first and last rows of its ``scale_inv``, which the finishing
    call converts to scales in place; between the two calls they hold the
    shard's partial maxima, for the caller's exchange to replace with the
    full ones."""

    def __init__(self, table, outputs, edges, bm, bn, device, keep):
        self.table, self.outputs, self.edges = table, outputs, edges
        self.bm, self.bn, self.device, self._keep = bm, bn, device, keep


def row_shards_begin(xs: Sequence, block_size=(128, 128), row_phases=None, maxima_event=None,
                     workspace=None) -> RowShards:
    """Partial maxima of the shards' edge rows, then the whole tile rows
    between them quantized in one pass (``fp8bq_row_shards_begin``).  Each
    shard is a BF16 [M, N] GPU tensor of whole rows whose first row sits at
    ``row_phases[i]`` inside a tile row (default 0).  ``maxima_event``
    (a ``torch.cuda.Event``) is recorded on the current stream once the
    maxima are enqueued.  An empty shard gets a [0, TN] scale_inv."""
    import torch

    bm, bn = block_shape(block_size)
    xs = list(xs)
    phases = [int(p) for p in (row_phases if row_phases is not None else [0] * len(xs))]
    if len(phases) != len(xs):
        raise ValueError("row_phases must hold one row phase per shard")
    dev = xs[0].device if xs else None
    table = (RowShardEntry * len(xs))()
    outputs, edges = [], []
    for e, x, rp in zip(table, xs, phases):
        _check_input(x)
        if x.device != dev:
            raise ValueError("all shards of one call must be on the same device")
        M, N = x.shape
        TMl, TN = local_grid(M, N, bm, bn, (rp, 0)) if M else (0, -(-N // bn))
        top, bottom = row_shard_edges(M, bm, rp)
        q = torch.empty((M, N), dtype=torch.float8_e4m3fn, device=dev)
        s = torch.empty((TMl, TN), dtype=torch.float32, device=dev)
        ta = s[0] if top and N else None
        ba = s[TMl - 1] if bottom and N else None
        e.x, e.q, e.scale_inv, e.M, e.N, e.row_phase = x.data_ptr(), q.data_ptr(), s.data_ptr(), M, N, rp
        e.top_amax = ta.data_ptr() if ta is not None else None
        e.bottom_amax = ba.data_ptr() if ba is not None else None
        outputs.append((q, s))
        edges.append((ta, ba))
    if not xs:
        return RowShards(table, [], [], bm, bn, dev, ())
    lib = load_library()
    need = int(lib.fp8bq_many_workspace_bytes(len(xs)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        ev = maxima_event.cuda_event if maxima_event is not None else None
        if maxima_event is not None and ev == 0:   # torch creates its event on first record
            maxima_event.record()
            ev = maxima_event.cuda_event
        _check("fp8bq_row_shards_begin",
               lib.fp8bq_row_shards_begin(table, len(xs), bm, bn, ws_ptr, ws_bytes, ev, _stream(dev)))
    return RowShards(table, outputs, edges, bm, bn, dev, (xs, workspace))


def row_shards_finish(state: RowShards) -> List:
    """The edge rows quantized with the maxima now in ``state.edges``
    (``fp8bq_row_shards_finish``).  Returns (q, scale_inv) per shard."""
    import torch

    if state.outputs:
        with torch.cuda.device(state.device):
            _check("fp8bq_row_shards_finish",
                   load_library().fp8bq_row_shards_finish(state.table, len(state.outputs), state.bm,
                                                          state.bn, _stream(state.device)))
    return state.outputs


def quantize_row_shards(xs: Sequence, block_size=(128, 128), row_phases=None, exchange=None) -> List:
    """Quantize-before-gather of row shards: ``row_shards_begin``, then
    ``exchange(edges)`` (which replaces, in place, each edge's maxima by the
    max over the shards sharing that tile row; default: nothing, each shard
    alone), then ``row_shards_finish``.  Returns (q, scale_inv) per shard."""
    state = row_shards_begin(xs, block_size, row_phases)
    if exchange is not None:
        exchange(state.edges)
    return row_shards_finish(state)


def set_resident_wait_us(microseconds: int) -> None:
    """Longest wait of a workgroup of the one-scale-per-tensor kernel for the
    tensor-wide maximum before it computes that maximum itself
    (``fp8bq_set_resident_wait_us``; process-wide, default 2000 us)."""
    _check("fp8bq_set_resident_wait_us", load_library().fp8bq_set_resident_wait_us(int(microseconds)))


def encode_e4m3(y):
    """The final cast alone: float32 GPU tensor -> e4m3fn codes (uint8), clamped to +-448."""
    import torch

    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous():
        raise TypeError("y must be a contiguous float32 GPU tensor")
    q = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    with torch.cuda.device(y.device):
        _check("fp8bq_encode_e4m3",
               load_library().fp8bq_encode_e4m3(y.data_ptr(), q.data_ptr(), y.numel(),
                                                _stream(y.device)))
    return q


__all__ = [
    "DqEntry", "EXPORTS", "Fp8bqError", "TensorEntry", "block_shape", "dequantize",
    "dequantize_many", "encode_e4m3",
    "load_library", "local_grid", "quantize_with_amax", "quantize_with_amax_many", "tile_amax",
    "tile_amax_many", "ShardEntry",
    "make_entries", "quantize", "quantize_many", "quantize_many_noalloc", "scale_shape",
    "set_resident_wait_us",
    "workspace_bytes",
]
