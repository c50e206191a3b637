"""CPU oracle for blockwise FP8 (OCP e4m3fn) weight quantization.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The GPU library never imports, links or calls it, and this
package imports nothing from the GPU library: the two share no code.

What it computes (the blockwise cast described on the documentation page
"fp8_kernel.py — FP8 量化内核" for verl/utils/kernel/fp8_kernel.py, section 2,
the Triton implementation, and its entry point in section 1): an [M, N] BF16
matrix is cut into [bm, bn] tiles; per tile the largest magnitude is floored
at ``eps``, divided by 448 to give the stored descale ``s``; every element is
multiplied by ``1/s``, clamped to +-448 and rounded to float8 e4m3fn.

Every floating-point step is done in float64 on values that are exactly
representable in float32, then rounded once to float32.  For a single
division or multiplication of float32 operands this equals the correctly
rounded float32 result (53 >= 2*24 + 2 bits, so the double rounding is
innocuous), which is the precision the method runs in.

Modules
-------
``e4m3fn``     the 8-bit format: decode, scalar and numpy encoders.
``fp32``       float32 rounding helpers and BF16 widening.
``blockwise``  the tile pipeline: a pure-Python scalar version for tiny
               inputs and a numpy version (per tile row) for larger ones;
               dequantization (decode(q) * s, to float32 or BF16); partial
               tile maxima of a shard and quantization with given maxima.
"""

from .blockwise import (  # noqa: F401
    EPS,
    E4M3_MAX,
    dequantize,
    local_grid,
    quantize,
    quantize_with_amax,
    quantize_scalar,
    quantize_tile,
    tile_amax,
    tile_scale,
    tile_grid,
)
from .e4m3fn import decode, decode_np, encode, encode_np  # noqa: F401
from .fp32 import bf16_bits_to_f64, fl32, fl32_np  # noqa: F401
