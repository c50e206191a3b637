"""The device code the build emits, read from its own gfx950 assembly (CPU
only): the numerics flags took effect in every kernel.

  * every kernel keeps fp32 denormals (no flush-to-zero mode);
  * every kernel that turns a tile maximum into s = a/448 and r = 1/s runs
    the correctly rounded division sequence (v_div_scale / v_div_fmas /
    v_div_fixup), not a bare reciprocal;
  * quantizers convert with the gfx950 OCP e4m3 instruction, dequantizers
    decode with its inverse;
  * no packed fp32 arithmetic is emitted anywhere.
"""

import re
import subprocess

import pytest

from fp8_blockwise_weight_amd import build as fb


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "fp8bq-gfx950.s"
    cmd = [c for c in fb.command(str(out)) if c not in ("-shared", "-fPIC")]
    cmd[1:1] = ["-S", "--cuda-device-only"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    return out.read_text()


def _bodies(text):
    """Kernel name -> its instructions (entry label to the function's end)."""
    return {m.group(1): m.group(2)
            for m in re.finditer(r"^(_ZN5fp8bq\w+):(.*?)^\.Lfunc_end\d+:", text, re.M | re.S)}


def _descriptors(text):
    """Kernel name -> its .amdhsa_kernel descriptor block."""
    return {m.group(1): m.group(2)
            for m in re.finditer(r"^\s*\.amdhsa_kernel (\S+)$(.*?)^\s*\.end_amdhsa_kernel", text,
                                 re.M | re.S)}


def test_every_kernel_keeps_fp32_denormals(asm):
    desc = _descriptors(asm)
    assert len(desc) >= 20
    for name, block in desc.items():
        mode = re.search(r"\.amdhsa_float_denorm_mode_32 (\d)", block)
        assert mode and mode.group(1) == "3", name


def test_no_packed_fp32_arithmetic(asm):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)


def test_scale_kernels_divide_correctly_rounded_and_encode_e4m3(asm):
    bodies = _bodies(asm)
    assert len(bodies) >= 20
    divides = [n for n in bodies if re.search(r"quantize_one|quantize_group|quantize_flat|big_reduce|"
                                              r"big_group_reduce|big_quant|big_group_quant|"
                                              r"finalize_scales|resident_quant|shard_group_wide", n)]
    assert len(divides) >= 15
    for n in divides:
        b = bodies[n]
        for op in ("v_div_scale_f32", "v_div_fmas_f32", "v_div_fixup_f32"):
            assert op in b, (n, op)
    for n in bodies:
        if re.search(r"quantize_one|quantize_group|quantize_flat|big_quant|big_group_quant|"
                     r"shard_(small|rows|group)ILi1|shard_group_wide|encode_e4m3|resident_quant", n):
            assert "v_cvt_pk_fp8_f32" in bodies[n], n
        if "dequant" in n:
            assert "v_cvt_pk_f32_fp8" in bodies[n], n
