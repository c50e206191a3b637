"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each ``pin_*`` function raises (AssertionError or the oracle's own error) when
the oracle disagrees with something the format, IEEE arithmetic or the
method's definition fixes independently of it:

* a library routine (torch's CPU cast to float8_e4m3fn and back);
* exact rational arithmetic with brute-force nearest-value search
  (``bruteforce``);
* the format's printed special values and hand-derived cases
  (``tests/golden``);
* closed-form invariants of the method (a non-zero tile reaches +-448, an
  all-zero tile takes the eps scale, e4m3 multiples round-trip exactly, the
  error stays within half an e4m3 ulp, monotonicity, tile independence).

``quick=True`` selects smaller samples; the mutation tests run every pin in
quick mode against oracles with a planted mistake.
"""

import math
import os
from fractions import Fraction

import numpy as np
import torch

import bruteforce as bf
import oracle
from oracle import e4m3fn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32)


def _bits_of(vals_f32) -> np.ndarray:
    """BF16 patterns of float32 values that are BF16-exact."""
    b = _f32(vals_f32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value is not BF16-exact"
    return (b >> 16).astype(np.uint16)


def _rng(seed):
    return np.random.default_rng(seed)


def _random_bf16(rng, shape, std=0.02) -> np.ndarray:
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * std)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def encoder_probe_values(quick: bool) -> np.ndarray:
    """float32 values that exercise every rounding decision of the encoder."""
    pos = [float(v) for v in bf.E4M3_POS_VALUES]
    mids = [(pos[i] + pos[i + 1]) / 2 for i in range(len(pos) - 1)]   # exact in float32
    vals = set(pos) | set(mids)
    for m in mids:
        lo = hi = np.float32(m)
        for _ in range(2):
            lo = np.nextafter(lo, np.float32(0), dtype=np.float32)
            hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
            vals.update([float(lo), float(hi)])
    rng = _rng(7)
    n = 2000 if quick else 20000
    vals.update(float(v) for v in _f32(np.exp2(rng.uniform(-14.0, math.log2(448.0), n))))
    vals.update([1e-45, 1e-40, 2.0 ** -126, 2.0 ** -10, 2.0 ** -11])
    vals = sorted(v for v in vals if v <= 448.0)
    arr = _f32(vals)
    return np.concatenate([arr, -arr, _f32([0.0, -0.0])])


# ---------------------------------------------------------------- the format

def pin_decode_matches_torch(quick=True):
    """Decoding all 256 codes agrees with torch's float8_e4m3fn -> float32 cast."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mine = np.array([oracle.decode(int(c)) for c in codes])
    mine_np = oracle.decode_np(codes)
    for got in (mine, mine_np):
        both_nan = np.isnan(ref) & np.isnan(got)
        assert np.all(both_nan | (ref == got)), "decode disagrees with torch"
        assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def pin_format_golden(quick=True):
    """The format's special values (tests/golden/e4m3fn_format_values.txt)."""
    for code_s, val_s, *_ in _golden_rows("e4m3fn_format_values.txt"):
        code = int(code_s, 16)
        val = float(val_s)
        got = oracle.decode(code)
        if math.isnan(val):
            assert math.isnan(got), code_s
            continue
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code_s
        assert oracle.encode(val) == code, code_s
        assert int(oracle.encode_np([val])[0]) == code, code_s


def pin_encoder_bruteforce(quick=True):
    """Both encoders equal the brute-force nearest code (ties to even) on every
    value, midpoint and near-midpoint of the grid, plus random values."""
    vals = encoder_probe_values(quick)
    if quick:
        vals = vals[:: max(1, len(vals) // 3000)]
    got_np = oracle.encode_np(vals.astype(np.float64))
    for v, g in zip(vals, got_np):
        want = bf.nearest_e4m3_code(v)
        assert int(g) == want, (float(v), int(g), want)
        assert oracle.encode(float(v)) == want, (float(v), want)


def pin_encoder_matches_torch(quick=True):
    """The numpy encoder equals torch's CPU float32 -> float8_e4m3fn cast."""
    vals = encoder_probe_values(quick)
    rng = _rng(11)
    n = 200_000 if quick else 2_000_000
    extra = _f32(np.exp2(rng.uniform(-30, math.log2(448.0), n)) * rng.choice([-1.0, 1.0], n))
    vals = np.concatenate([vals, extra])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode_np(vals.astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def pin_ties_golden(quick=True):
    """Hand-listed midpoints go to the even code through a unit-scale tile."""
    rows = _golden_rows("unit_scale_ties.txt")
    vals = [float(r[0]) for r in rows]
    want = [int(r[1], 16) for r in rows]
    tile = _bits_of([448.0] + vals)[None, :]
    q, s = oracle.quantize(tile, 1, tile.shape[1])
    assert float(s[0, 0]) == 1.0
    assert int(q[0, 0]) == 0x7E
    assert [int(c) for c in q[0, 1:]] == want
    qs, ss = oracle.quantize_scalar(tile.ravel().tolist(), 1, tile.shape[1], 1, tile.shape[1])
    assert qs[1:] == want and ss[0] == 1.0


# ---------------------------------------------------------------- the scale

def pin_scale_exhaustive_bf16(quick=True):
    """For every finite positive BF16 maximum (and zero), (s, r) equal the
    exact-arithmetic nearest float32 of max(amax, eps)/448 and of 1/s."""
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    if quick:
        bits = bits[::37]
    amax = oracle.bf16_bits_to_f64(bits)
    s_np, r_np = oracle.blockwise.tile_scales_np(amax)
    eps = bf.frac_of_f32(oracle.EPS)
    for i, b in enumerate(bits):
        a = max(bf.bf16_frac(int(b)), eps)
        s = bf.nearest_f32(a / 448)
        r = bf.nearest_f32(1 / Fraction(float(s)))
        assert s_np[i] == float(s) and r_np[i] == float(r), (hex(int(b)), s_np[i], float(s))
        if i % 50 == 0:
            s2, r2 = oracle.tile_scale(float(amax[i]))
            assert (s2, r2) == (float(s), float(r))


def pin_scale_golden(quick=True):
    """Hand-derived scales (tests/golden/hand_derived_cases.txt)."""
    for amax_s, bits_s, val_s, *_ in _golden_rows("hand_derived_cases.txt"):
        amax = float(amax_s)
        s, _ = oracle.tile_scale(amax)
        s_np, _ = oracle.blockwise.tile_scales_np(np.array([amax]))
        want = float(np.array([int(bits_s, 16)], dtype=np.uint32).view(np.float32)[0])
        assert s == want == float(val_s) == s_np[0], (amax_s, s, want)
        tile = np.zeros((2, 2), dtype=np.uint16)
        tile[1, 1] = _bits_of([amax])[0]
        q, sc = oracle.quantize(tile, 2, 2)
        assert float(sc[0, 0]) == want


# ---------------------------------------------------------------- whole tiles

def pin_tiny_bruteforce(quick=True):
    """Every tiny shape and block (M, N in 1..6; bm, bn in 1..4): exact
    arithmetic == scalar oracle == numpy oracle, on random, zero-holding and
    tie-holding inputs."""
    rng = _rng(3)
    shapes = [(M, N, bm, bn) for M in range(1, 7) for N in range(1, 7)
              for bm in range(1, 5) for bn in range(1, 5)]
    if quick:
        shapes = shapes[::23]
    for k, (M, N, bm, bn) in enumerate(shapes):
        kind = k % 3
        if kind == 0:
            x = _random_bf16(rng, (M, N), std=rng.choice([1e-3, 0.02, 3.0]))
        elif kind == 1:
            x = _random_bf16(rng, (M, N))
            x[rng.random((M, N)) < 0.4] = 0
            x[rng.random((M, N)) < 0.1] = 0x8000        # -0.0
        else:
            ties = _f32([1.0625, -1.1875, 0.0029296875, 248.0, -400.0, 432.0, 448.0, 2.0 ** -10])
            x = _bits_of(rng.choice(ties, size=(M, N)))
        q_ex, s_ex = bf.quantize_exact(x, bm, bn, oracle.EPS)
        q_np, s_np = oracle.quantize(x, bm, bn)
        q_sc, s_sc = oracle.quantize_scalar(x.ravel().tolist(), M, N, bm, bn)
        assert np.array_equal(q_np, q_ex), (M, N, bm, bn, kind)
        assert np.array_equal(s_np.view(np.uint32), s_ex.view(np.uint32)), (M, N, bm, bn)
        assert np.array_equal(np.array(q_sc, dtype=np.uint8).reshape(M, N), q_ex)
        assert np.array_equal(_f32(s_sc).reshape(s_ex.shape).view(np.uint32), s_ex.view(np.uint32))


def pin_anchor_sweep(quick=True):
    """[1, n] rows holding an anchor maximum and a sweep of BF16 values below
    it: numpy oracle == exact arithmetic (covers scaled values landing near
    e4m3 rounding boundaries)."""
    rng = _rng(5)
    n_rows = 6 if quick else 40
    rows = []
    for _ in range(n_rows):
        anchor = np.float32(np.exp2(rng.uniform(-20, 20)))
        anchor_bits = _bits_of([np.float32(torch.tensor(float(anchor)).to(torch.bfloat16).float())])[0]
        a = float(oracle.bf16_bits_to_f64([anchor_bits])[0])
        # every BF16 pattern below the anchor's magnitude, thinned to a sample
        cand = np.arange(0, anchor_bits, max(1, anchor_bits // 300), dtype=np.uint16)
        sign = rng.integers(0, 2, cand.size).astype(np.uint16) << 15
        row = np.concatenate([[anchor_bits], cand | sign]).astype(np.uint16)
        rows.append((row, a))
    for row, _ in rows:
        x = row[None, :]
        q_np, s_np = oracle.quantize(x, 1, x.shape[1])
        codes, s = bf.quantize_tile_exact([int(b) for b in row], oracle.EPS)
        assert float(s_np[0, 0]) == float(s)
        assert np.array_equal(q_np[0], np.array(codes, dtype=np.uint8))


def pin_double_rounding_cases(quick=True):
    """Inputs whose scaled value x*r rounds (in float32) exactly onto an e4m3
    midpoint without being on it: the float32 rounding of the product decides
    the code.  Oracle == exact arithmetic on every such case found."""
    pos = np.array([float(v) for v in bf.E4M3_POS_VALUES])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = _rng(19)
    eps = bf.frac_of_f32(oracle.EPS)
    found = 0
    for _ in range(12 if quick else 60):
        ab = int(rng.integers(0x2000, 0x6000))
        a = max(bf.bf16_frac(ab), eps)
        r = float(bf.nearest_f32(1 / Fraction(float(bf.nearest_f32(a / 448)))))
        xb = np.arange(1, ab, dtype=np.uint16)
        x = oracle.bf16_bits_to_f64(xb)
        p = x * r                                   # exact in float64 (8 x 24 bits)
        y = p.astype(np.float32).astype(np.float64)
        hit = xb[np.isin(y, mids) & (p != y)][:24]
        if hit.size == 0:
            continue
        found += hit.size
        row = np.concatenate([[ab], hit, hit | 0x8000]).astype(np.uint16)
        codes, s = bf.quantize_tile_exact([int(b) for b in row], oracle.EPS)
        q_np, s_np = oracle.quantize(row[None, :], 1, row.size)
        assert float(s_np[0, 0]) == float(s)
        assert np.array_equal(q_np[0], np.array(codes, dtype=np.uint8)), hex(ab)
        q_sc, _ = oracle.quantize_scalar(row.tolist(), 1, row.size, 1, row.size)
        assert q_sc == codes
    assert found > 0, "no double-rounding case found; widen the search"


# ---------------------------------------------------------------- invariants

def _inv_inputs(quick):
    """(name, bits, bm, bn) cases for the invariant checks."""
    rng = _rng(9)
    cases = []
    # C1-like: outliers in tile (0,0), zero tile (1,1)
    x = (torch.from_numpy(rng.standard_normal((256, 256)).astype(np.float32)) * 0.02)
    x[5, 7], x[100, 3], x[64, 127] = 5.0, -5.0, 5.0
    x[128:, 128:] = 0
    cases.append(("c1like", x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), 128, 128))
    shapes = [(77, 128), (200, 300)] if quick else [(77, 128), (1000, 3000), (333, 517)]
    for M, N in shapes:
        x = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)) * 0.02
        lap = torch.from_numpy(rng.laplace(0, 0.2, (M, N)).astype(np.float32))
        x = torch.where(torch.from_numpy(rng.random((M, N)) < 0.1), lap, x)
        x[0] = 0
        bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        for bm, bn in ((128, 128), (64, 64), (1, 128), (3, 5)):
            cases.append((f"{M}x{N}/{bm}x{bn}", bits, bm, bn))
    return cases


def _tiles(M, N, bm, bn):
    TM, TN = oracle.tile_grid(M, N, bm, bn)
    for ti in range(TM):
        for tj in range(TN):
            yield ti, tj, slice(ti * bm, min(M, (ti + 1) * bm)), slice(tj * bn, min(N, (tj + 1) * bn))


def pin_invariants(quick=True):
    """I1 max |q| is 448 on tiles above eps (at the max element, with its
    sign); I2 zero tiles take fl32(eps/448) and code 0; I4 error within half
    an e4m3 ulp times s (plus float32 rounding of s, r, y); I5 monotone and
    sign-preserving; I6 scale matches an independent torch.amax; I8 no NaN
    codes."""
    eps32 = float(np.float32(oracle.EPS))
    zero_scale = float(np.float32(np.float64(np.float32(oracle.EPS)) / 448.0))
    for name, bits, bm, bn in _inv_inputs(quick):
        M, N = bits.shape
        q, s = oracle.quantize(bits, bm, bn)
        xf = oracle.bf16_bits_to_f64(bits)
        assert not np.any((q == 0x7F) | (q == 0xFF)), name                       # I8
        dq = oracle.decode_np(q)
        xt = torch.from_numpy(xf)
        for ti, tj, rs, cs in _tiles(M, N, bm, bn):
            tx, tq, tdq = xf[rs, cs], q[rs, cs], dq[rs, cs]
            sc = float(s[ti, tj])
            amax = float(torch.amax(torch.abs(xt[rs, cs])))                        # I6
            assert sc == float(np.float32(max(amax, eps32) / 448.0)), name
            if amax >= eps32:                                                      # I1
                assert np.max(np.abs(tdq)) == 448.0, (name, ti, tj)
                k = np.unravel_index(np.argmax(np.abs(tx)), tx.shape)
                assert int(tq[k]) == (0xFE if tx[k] < 0 else 0x7E), (name, ti, tj)
            if amax == 0:                                                          # I2
                assert sc == zero_scale, name
                assert np.all((tq & 0x7F) == 0), name
            # I4: in float64, |x - decode(q) s| <= ulp(y)/2 * s + 2**-22 |x|
            y = np.abs(tx) / sc
            e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
            ulp = np.where(y >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
            err = np.abs(tx - tdq * sc)
            assert np.all(err <= 0.5 * ulp * sc + 2.0 ** -22 * np.abs(tx)), (name, ti, tj)
            # I5: sign kept, order kept
            assert np.array_equal(np.signbit(tx), (tq & 0x80) != 0), name
            order = np.argsort(tx, axis=None, kind="stable")
            assert np.all(np.diff(tdq.ravel()[order]) >= 0), name


def pin_roundtrip_e4m3_multiples(quick=True):
    """I3: a tile of e4m3 values c times s0 (s0 = 2**k or 3 * 2**k) holding a
    +-448 entry has scale exactly s0, codes exactly c, and decodes exactly."""
    rng = _rng(13)
    pos = np.array([float(v) for v in bf.E4M3_POS_VALUES])
    ks = range(-30, 20, 7 if quick else 1)
    for k in ks:
        for mult in (1.0, 3.0):
            s0 = mult * 2.0 ** k
            c = rng.choice(pos, size=(4, 16)) * rng.choice([-1.0, 1.0], size=(4, 16))
            c[rng.integers(0, 4), rng.integers(0, 16)] = 448.0 * rng.choice([-1.0, 1.0])
            x = c * s0
            bits = _bits_of(_f32(x))
            q, s = oracle.quantize(bits, 4, 16)
            assert float(s[0, 0]) == s0, (k, mult)
            assert np.array_equal(oracle.decode_np(q), c), (k, mult)
            assert np.array_equal(oracle.decode_np(q) * float(s[0, 0]), x)


def pin_tile_independence(quick=True):
    """I7: a tile-aligned sub-matrix quantizes to the same bytes and scales."""
    rng = _rng(17)
    bits = _random_bf16(rng, (300, 520))
    for bm, bn in ((128, 128), (64, 64), (1, 128), (7, 9)):
        q, s = oracle.quantize(bits, bm, bn)
        r0, c0 = bm * 1, bn * 2
        q2, s2 = oracle.quantize(bits[r0:, c0:].copy(), bm, bn)
        assert np.array_equal(q[r0:, c0:], q2)
        assert np.array_equal(s[1:, 2:], s2)


# ---------------------------------------------------------------- dequantization

def pin_dequant_bruteforce(quick=True):
    """decode(q) * s rounded once to float32: equal to exact arithmetic with a
    nearest-float32 search; the BF16 output equals torch's CPU
    float32 -> bfloat16 cast (a library routine)."""
    rng = _rng(23)
    n = 300 if quick else 3000
    codes = rng.integers(0, 256, (1, n)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E                     # no NaN codes
    bm, bn = 1, 1
    scales = _f32(np.exp2(rng.uniform(-40, 40, (1, n))))
    got = oracle.dequantize(codes, scales, bm, bn, "f32")
    got16 = oracle.dequantize(codes, scales, bm, bn, "bf16")
    for j in range(n):
        v = bf.E4M3_POS_VALUES[int(codes[0, j]) & 0x7F] * (-1 if codes[0, j] & 0x80 else 1)
        want = bf.nearest_f32(v * Fraction(float(scales[0, j])), negative_zero=bool(codes[0, j] & 0x80))
        assert got[0, j] == float(want), (int(codes[0, j]), float(scales[0, j]))
    ref16 = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ref16.astype(np.float64), got16)
    big = _f32(np.exp2(rng.uniform(-120, 120, 200_000 if not quick else 20_000)) *
               rng.choice([-1.0, 1.0], 200_000 if not quick else 20_000))
    ref = torch.from_numpy(big).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.blockwise.round_to_bf16(big.astype(np.float64)), ref)


def pin_dequant_roundtrip(quick=True):
    """I3 through dequantization: e4m3 multiples come back exactly (float32
    and BF16); I4: the float32 dequantized error stays within half an e4m3
    ulp of the scaled value times s (plus float32 rounding)."""
    rng = _rng(29)
    pos = np.array([float(v) for v in bf.E4M3_POS_VALUES])
    for k in range(-20, 20, 9 if quick else 3):
        c = rng.choice(pos, size=(8, 32)) * rng.choice([-1.0, 1.0], size=(8, 32))
        c[0, 0] = 448.0
        x = c * 2.0 ** k
        bits = _bits_of(_f32(x))
        q, s = oracle.quantize(bits, 8, 32)                  # one tile holding the 448
        for out in ("f32", "bf16"):
            assert np.array_equal(oracle.dequantize(q, s, 8, 32, out), x), (k, out)
    for name, bits, bm, bn in _inv_inputs(True)[:3]:
        q, s = oracle.quantize(bits, bm, bn)
        xf = oracle.bf16_bits_to_f64(bits)
        xh = oracle.dequantize(q, s, bm, bn, "f32")
        s_full = np.repeat(np.repeat(s.astype(np.float64), bm, 0)[:bits.shape[0]], bn, 1)[:, :bits.shape[1]]
        y = np.abs(xf) / s_full
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        ulp = np.where(y >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
        assert np.all(np.abs(xf - xh) <= 0.5 * ulp * s_full + 2.0 ** -21 * np.abs(xf)), name


# ---------------------------------------------------------------- shards

def shard_quantize(bits, bm, bn, row_cuts, col_cuts, amax_fn, quant_fn):
    """Quantize a matrix shard by shard: partial maxima per shard, combined by
    max over the shards that share a tile, then each shard quantized with the
    combined maxima.  Returns the re-assembled (q, scale_inv)."""
    M, N = bits.shape
    TM, TN = oracle.tile_grid(M, N, bm, bn)
    rb = [0] + list(row_cuts) + [M]
    cb = [0] + list(col_cuts) + [N]
    full = np.zeros((TM, TN))
    parts = []
    for i in range(len(rb) - 1):
        for j in range(len(cb) - 1):
            r0, r1, c0, c1 = rb[i], rb[i + 1], cb[j], cb[j + 1]
            if r0 == r1 or c0 == c1:
                continue
            rp, cp = r0 % bm, c0 % bn
            a = amax_fn(np.ascontiguousarray(bits[r0:r1, c0:c1]), bm, bn, rp, cp)
            t0, u0 = r0 // bm, c0 // bn
            view = full[t0:t0 + a.shape[0], u0:u0 + a.shape[1]]
            np.maximum(view, a, out=view)
            parts.append((r0, r1, c0, c1, rp, cp, t0, u0))
    q = np.zeros((M, N), dtype=np.uint8)
    s_out = np.zeros((TM, TN), dtype=np.float32)
    for r0, r1, c0, c1, rp, cp, t0, u0 in parts:
        TMl, TNl = oracle.local_grid(r1 - r0, c1 - c0, bm, bn, rp, cp)
        qs, ss = quant_fn(np.ascontiguousarray(bits[r0:r1, c0:c1]), bm, bn,
                          full[t0:t0 + TMl, u0:u0 + TNl], rp, cp)
        q[r0:r1, c0:c1] = qs
        s_out[t0:t0 + TMl, u0:u0 + TNl] = ss
    return q, s_out


def pin_shards_equal_whole(quick=True):
    """Sharded quantization (partial maxima exchanged as a max over the shards
    sharing a tile, cuts anywhere, including inside tiles) equals quantizing
    the whole matrix; and whole-matrix maxima reproduce ``quantize``."""
    rng = _rng(37)
    cases = [(300, 520, 128, 128), (77, 200, 64, 64), (129, 257, 1, 128), (50, 60, 7, 9),
             (200, 300, 200, 300)]
    for M, N, bm, bn in cases[: 3 if quick else None]:
        bits = _random_bf16(rng, (M, N))
        q_ref, s_ref = oracle.quantize(bits, bm, bn)
        a = oracle.tile_amax(bits, bm, bn)
        q1, s1 = oracle.quantize_with_amax(bits, bm, bn, a)
        assert np.array_equal(q1, q_ref) and np.array_equal(s1.view(np.uint32), s_ref.view(np.uint32))
        for _ in range(2 if quick else 6):
            rc = sorted(set(int(v) for v in rng.integers(1, M, rng.integers(0, 4))))
            cc = sorted(set(int(v) for v in rng.integers(1, N, rng.integers(0, 3))))
            q2, s2 = shard_quantize(bits, bm, bn, rc, cc, oracle.tile_amax, oracle.quantize_with_amax)
            assert np.array_equal(q2, q_ref), (M, N, bm, bn, rc, cc)
            assert np.array_equal(s2.view(np.uint32), s_ref.view(np.uint32)), (M, N, bm, bn, rc, cc)


PINS = [
    pin_decode_matches_torch,
    pin_format_golden,
    pin_encoder_bruteforce,
    pin_encoder_matches_torch,
    pin_ties_golden,
    pin_scale_exhaustive_bf16,
    pin_scale_golden,
    pin_tiny_bruteforce,
    pin_anchor_sweep,
    pin_double_rounding_cases,
    pin_invariants,
    pin_roundtrip_e4m3_multiples,
    pin_tile_independence,
    pin_dequant_bruteforce,
    pin_dequant_roundtrip,
    pin_shards_equal_whole,
]
