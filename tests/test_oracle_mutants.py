"""Plant plausible mistakes in the CPU oracle and check that its pins catch each one.

Every mutant below patches the oracle (never the GPU path) for the duration
of one test and runs the pins in quick mode; at least one pin must fail.
This shows the pins are strong enough that a dropped term, a wrong rounding
or a mis-indexed tile in the oracle would not go unnoticed.
"""

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle import blockwise, e4m3fn
from oracle.fp32 import fl32


def _patch_encoders(mp, enc, enc_np):
    for mod in (oracle, e4m3fn, blockwise):
        mp.setattr(mod, "encode", enc, raising=False)
        mp.setattr(mod, "encode_np", enc_np, raising=False)


def _patch_scales(mp, scalar, vector):
    mp.setattr(blockwise, "tile_scale", scalar)
    mp.setattr(oracle, "tile_scale", scalar)
    mp.setattr(blockwise, "tile_scales_np", vector)


def m_single_division(mp):
    """Reciprocal taken as 448/amax instead of 1/s (the two-division order dropped)."""
    def scalar(amax, eps=oracle.EPS):
        a = max(amax, fl32(eps))
        return fl32(a / 448.0), fl32(448.0 / a)

    def vector(amax, eps=oracle.EPS):
        a = np.maximum(amax, fl32(eps))
        return ((a / 448.0).astype(np.float32).astype(np.float64),
                (448.0 / a).astype(np.float32).astype(np.float64))
    _patch_scales(mp, scalar, vector)


def m_no_eps_floor(mp):
    """The eps floor dropped: an all-zero tile divides by zero."""
    def scalar(amax, eps=oracle.EPS):
        s = fl32(amax / 448.0)
        return s, (fl32(1.0 / s) if s else float("inf"))

    def vector(amax, eps=oracle.EPS):
        with np.errstate(divide="ignore"):
            s = (amax / 448.0).astype(np.float32).astype(np.float64)
            return s, (1.0 / s).astype(np.float32).astype(np.float64)
    _patch_scales(mp, scalar, vector)


def m_store_reciprocal(mp):
    """The stored descale is 1/s instead of s."""
    orig_s, orig_v = blockwise.tile_scale, blockwise.tile_scales_np

    def scalar(amax, eps=oracle.EPS):
        _, r = orig_s(amax, eps)
        return r, r

    def vector(amax, eps=oracle.EPS):
        _, r = orig_v(amax, eps)
        return r, r
    _patch_scales(mp, scalar, vector)


def m_ties_away(mp):
    """Encoder rounds half away from zero instead of half to even."""
    orig_np = e4m3fn.encode_np

    def enc_np(y):
        y = np.asarray(y, dtype=np.float64)
        out = orig_np(y)
        # redo the rounding with floor(x + 0.5)
        a = np.abs(y)
        sub = np.floor(a * 512.0 + 0.5).astype(np.int64)
        f, e = np.frexp(np.where(a < 2.0 ** -6, 1.0, a))
        e = e.astype(np.int64) - 1
        m = np.floor((2 * f - 1) * 8 + 0.5).astype(np.int64)
        e = e + (m == 8)
        m = np.where(m == 8, 0, m)
        mag = np.where(a < 2.0 ** -6, sub, ((e + 7) << 3) | m)
        return ((out & 0x80) | mag).astype(np.uint8)

    def enc(v):
        return int(enc_np(np.array([v]))[0])
    _patch_encoders(mp, enc, enc_np)


def m_lose_negative_zero(mp):
    """Encoder takes the sign from y < 0, so -0.0 and tiny negatives lose it."""
    orig_np = e4m3fn.encode_np

    def enc_np(y):
        y = np.asarray(y, dtype=np.float64)
        out = orig_np(y) & 0x7F
        return (out | np.where(y < 0, 0x80, 0)).astype(np.uint8)

    def enc(v):
        return int(enc_np(np.array([v]))[0])
    _patch_encoders(mp, enc, enc_np)


def m_subnormal_step(mp):
    """Subnormal grid taken as 2**-8 instead of 2**-9."""
    orig_np = e4m3fn.encode_np

    def enc_np(y):
        y = np.asarray(y, dtype=np.float64)
        out = orig_np(y)
        a = np.abs(y)
        sub = np.rint(a * 256.0).astype(np.int64)
        return np.where(a < 2.0 ** -6, (out & 0x80) | sub, out).astype(np.uint8)

    def enc(v):
        return int(enc_np(np.array([v]))[0])
    _patch_encoders(mp, enc, enc_np)


def m_decode_sign(mp):
    """Decoder ignores the sign bit."""
    orig, orig_np = e4m3fn.decode, e4m3fn.decode_np
    for mod in (oracle, e4m3fn):
        mp.setattr(mod, "decode", lambda c: orig(c & 0x7F), raising=False)
        mp.setattr(mod, "decode_np", lambda c: orig_np(np.asarray(c, dtype=np.uint8) & 0x7F), raising=False)


def m_amax_first_row_only(mp):
    """Tile maximum taken over the tile's first row only (a mis-indexed reduction)."""
    orig = blockwise.tile_row_amax
    mp.setattr(blockwise, "tile_row_amax", lambda x_abs, TN, bn: orig(x_abs[:1], TN, bn))


def m_amax_drops_last_row(mp):
    """Edge off-by-one: the tile maximum misses the tile's last row."""
    orig = blockwise.tile_row_amax
    mp.setattr(blockwise, "tile_row_amax",
               lambda x_abs, TN, bn: orig(x_abs[:-1] if len(x_abs) > 1 else x_abs, TN, bn))


def m_no_float32_product(mp):
    """The scaled value x*r is encoded from float64 without rounding to float32."""
    def sce(x, r_col):
        y = x * r_col
        y = np.minimum(np.maximum(y, -448.0), 448.0)
        return blockwise.encode_np(y)
    mp.setattr(blockwise, "scale_clamp_encode", sce)


def m_columns_shifted(mp):
    """Each element uses the reciprocal of the tile to its right (wrong column map)."""
    orig = blockwise.scale_clamp_encode

    def sce(x, r_col):
        return orig(x, np.roll(r_col, -1))
    mp.setattr(blockwise, "scale_clamp_encode", sce)


def m_dequant_divides(mp):
    """Dequantization divides by the descale instead of multiplying."""
    orig = blockwise.dequantize

    def deq(q, scale_inv, bm, bn, out="f32"):
        inv = (1.0 / np.asarray(scale_inv, dtype=np.float64)).astype(np.float32)
        return orig(q, inv, bm, bn, out)
    mp.setattr(blockwise, "dequantize", deq)
    mp.setattr(oracle, "dequantize", deq)


def m_bf16_truncates(mp):
    """BF16 output truncated (rounded toward zero) instead of rounded to nearest even."""
    def rt(y):
        y = np.asarray(y, dtype=np.float64)
        b = y.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        return b.view(np.float32).astype(np.float64)
    mp.setattr(blockwise, "round_to_bf16", rt)


def m_phase_ignored(mp):
    """Shard maxima computed as if every shard started on a tile boundary."""
    orig = blockwise.tile_amax

    def ta(x_bits, bm, bn, row_phase=0, col_phase=0):
        a = orig(x_bits, bm, bn, 0, 0)
        TM, TN = blockwise.local_grid(*np.asarray(x_bits).shape, bm, bn, row_phase, col_phase)
        out = np.zeros((TM, TN))
        out[:min(TM, a.shape[0]), :min(TN, a.shape[1])] = a[:TM, :TN]
        return out
    mp.setattr(blockwise, "tile_amax", ta)
    mp.setattr(oracle, "tile_amax", ta)


def m_reciprocal_not_rounded(mp):
    """The reciprocal 1/s kept in float64 instead of rounded to float32."""
    def scalar(amax, eps=oracle.EPS):
        a = max(amax, fl32(eps))
        s = fl32(a / 448.0)
        return s, 1.0 / s

    def vector(amax, eps=oracle.EPS):
        a = np.maximum(amax, fl32(eps))
        s = (a / 448.0).astype(np.float32).astype(np.float64)
        return s, 1.0 / s
    _patch_scales(mp, scalar, vector)


def m_grid_floor(mp):
    """Tile counts rounded down: a ragged last tile row or column is dropped."""
    mp.setattr(blockwise, "tile_grid", lambda M, N, bm, bn: (M // bm, N // bn))


MUTANTS = [
    m_single_division,
    m_no_eps_floor,
    m_store_reciprocal,
    m_ties_away,
    m_lose_negative_zero,
    m_subnormal_step,
    m_decode_sign,
    m_amax_first_row_only,
    m_amax_drops_last_row,
    m_no_float32_product,
    m_columns_shifted,
    m_dequant_divides,
    m_bf16_truncates,
    m_phase_ignored,
    m_reciprocal_not_rounded,
    m_grid_floor,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_mutant(mutant, monkeypatch):
    mutant(monkeypatch)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(quick=True)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught {mutant.__name__}"
