"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact in both outputs: every fp8 byte and every fp32 scale.  Small and
medium tensors are compared whole in this process; the full-size weight sets
(the 36-layer dense stack in the one grouped launch the benchmark times,
all 48 MoE layers, the 151937x4096 matrix at every block size), the 2^31+
element matrices and the one-scale-per-tensor cases are compared whole too,
every byte and scale, by the oracle running on the host's cores
(``oracle.pool``: slabs of whole tile rows, or two passes over pieces of
tiles too large for a slab).
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_weight_amd as fq
import oracle
from fp8_blockwise_weight_amd import workloads as wl
from gpu_helpers import (FullOracleCheck, assert_matches_oracle, assert_properties_gpu, bits_np,
                         codes_np, scales_bits, tile_amax_gpu)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BLOCKS = [(128, 128), (64, 64), (1, 128)]


def say(*a):
    print(*a, flush=True)


def bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


# ------------------------------------------------------------------ C1

def test_c1_matches_oracle_and_closed_forms(gpu_lib):
    (spec,) = wl.c1()
    x = wl.materialize(spec, DEV)
    q, s = fq.quantize(x, (128, 128))
    torch.cuda.synchronize()
    assert q.dtype == torch.float8_e4m3fn and q.shape == (256, 256)
    assert s.dtype == torch.float32 and s.shape == (2, 2)
    assert_matches_oracle(x, q, s, 128, 128, "C1")
    sh = s.cpu().numpy()
    assert sh[0, 0] == np.float32(5.0 / 448.0)
    assert sh[1, 1] == np.float32(np.float64(np.float32(1e-10)) / 448.0)
    codes = codes_np(q)
    xb = bits_np(x)
    outl = np.abs(oracle.bf16_bits_to_f64(xb[:128, :128])) == 5.0
    assert outl.sum() == 8
    assert set(np.unique(codes[:128, :128][outl])) <= {0x7E, 0xFE}
    assert np.all(codes[128:, 128:] == 0)


# ------------------------------------------------------------------ seeded fuzz over every path

def _fuzz_bits(rng, M, N, family):
    """BF16 bit patterns [M, N] of one value family (all finite)."""
    if family == "bits":                       # any finite BF16: exponents 0..254
        b = rng.integers(0, 1 << 16, (M, N), dtype=np.uint32).astype(np.uint16)
        exp = (b >> 7) & 0xFF
        b[exp == 0xFF] &= 0x807F                # exponent 255 (Inf/NaN) -> 0
        return b
    sigma = {"normal": 10.0 ** rng.uniform(-30, 30), "tiny": 1e-13, "unit": 1.0}[family]
    v = (rng.standard_normal((M, N)) * sigma).astype(np.float32)
    if rng.random() < 0.3:
        v[rng.integers(0, M, max(1, M // 10))] = 0.0      # zero rows
    b = v.view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)   # RNE to BF16
    return b


def test_seeded_fuzz_all_paths(gpu_lib):
    """160 seeded random configurations through fp8bq_quantize, each against
    the oracle bit for bit, then the same tensors per block size through
    fp8bq_quantize_many (equal to the single calls).  Shapes 1..600 with N
    8-aligned or not, the three vector block kinds and random blocks up to
    [300, 300] (register, loop-vector, element and two-pass bodies), x as a
    misaligned view in a third of the cases, and value families from random
    finite bit patterns to tiles below eps."""
    rng = np.random.default_rng(20240607)
    cases = []
    for i in range(160):
        M = int(rng.integers(1, 601))
        N = int(rng.integers(1, 76)) * 8 if rng.random() < 0.6 else int(rng.integers(1, 601))
        r = rng.random()
        if r < 0.35:
            block = BLOCKS[int(rng.integers(0, 3))]
        elif r < 0.5:
            block = (int(rng.integers(256, 301)), int(rng.integers(256, 301)))   # large tiles when M, N allow
        else:
            block = (int(rng.integers(1, 301)), int(rng.integers(1, 301)))
        family = ["normal", "bits", "tiny", "unit"][int(rng.integers(0, 4))]
        bits = _fuzz_bits(rng, M, N, family)
        off = int(rng.integers(1, 8)) if rng.random() < 0.33 else 0
        flat = np.zeros(M * N + 8, dtype=np.uint16)
        flat[off:off + M * N] = bits.reshape(-1)
        base = torch.from_numpy(flat.view(np.int16)).to(DEV).view(torch.bfloat16)
        x = base[off:off + M * N].view(M, N)
        what = f"fuzz[{i}] {M}x{N} block {block} {family} offset {off}"
        say(what)
        q, s = fq.quantize(x, block)
        assert_matches_oracle(x, q, s, *block, what)
        cases.append((x, block, q, s))
    by_block = {}
    for x, block, q, s in cases:
        by_block.setdefault(block, []).append((x, q, s))
    for block, items in by_block.items():
        outs = fq.quantize_many([x for x, _, _ in items], block)
        for (x, q, s), (qg, sg) in zip(items, outs):
            assert torch.equal(qg.view(torch.uint8), q.view(torch.uint8)), block
            assert torch.equal(sg.view(torch.int32), s.view(torch.int32)), block


# ------------------------------------------------------------------ shapes and tails

@pytest.mark.parametrize("bm,bn", BLOCKS)
def test_vector_kinds_small_shapes(gpu_lib, bm, bn):
    """Every tail combination around the 64/128-row and 128-column unit edges."""
    g = torch.Generator(device=DEV).manual_seed(1234 + bm)
    for M in (1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200, 257):
        for N in (8, 16, 120, 128, 136, 248, 256, 264, 384):
            say("case", bm, bn, M, N)
            x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
            q, s = fq.quantize(x, (bm, bn))
            assert_matches_oracle(x, q, s, bm, bn, f"{M}x{N}/{bm}x{bn}")


def test_general_tiny_exhaustive(gpu_lib):
    """All M, N in 1..6 and bm, bn in 1..4 (the element-wise kernel)."""
    g = torch.Generator(device=DEV).manual_seed(99)
    for M in range(1, 7):
        for N in range(1, 7):
            x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
            x[torch.rand((M, N), generator=g, device=DEV) < 0.2] = 0
            for bm in range(1, 5):
                for bn in range(1, 5):
                    q, s = fq.quantize(x, (bm, bn))
                    assert_matches_oracle(x, q, s, bm, bn, f"{M}x{N}/{bm}x{bn}")


@pytest.mark.parametrize("block", [(128, 128), (64, 64), (1, 128), (128, 64), (32, 32), (3, 5),
                                   (1, 1), (256, 256), (1, 4096)])
def test_general_path_odd_and_misaligned(gpu_lib, block):
    """N % 8 != 0, misaligned x or q, and block sizes without a vector kernel."""
    bm, bn = block
    g = torch.Generator(device=DEV).manual_seed(7)
    for M, N in ((300, 7), (129, 1001), (65, 3001), (200, 520)):
        say("case", block, M, N)
        big = (torch.randn(M * N + 8, generator=g, device=DEV) * 0.3).to(torch.bfloat16)
        for off in (0, 1, 3):
            x = big[off:off + M * N].view(M, N)   # off > 0: x not 16-byte aligned
            qbuf = torch.empty(M * N + 8, dtype=torch.uint8, device=DEV)
            q = qbuf[off:off + M * N].view(M, N)  # off > 0: q not 8-byte aligned
            s = torch.empty(fq.scale_shape(M, N, bm, bn), dtype=torch.float32, device=DEV)
            fq.quantize(x, block, out=(q, s))
            assert_matches_oracle(x, q, s, bm, bn, f"{M}x{N}/{block}/off{off}")


@pytest.mark.parametrize("block", [(1, 4096), (16, 1024), (128, 64), (8, 8), (1, 16384), (32, 512),
                                   (256, 256), (64, 512), (200, 200)])
def test_register_and_loop_tile_bodies(gpu_lib, block):
    """Blocks with 8-aligned columns: up to 16384 elements take the
    register-resident tile body, up to 65536 the two-pass vector body;
    ragged edges included."""
    bm, bn = block
    g = torch.Generator(device=DEV).manual_seed(17)
    for M, N in ((77, 128), (1000, 3000), (4097, 1008), (33, 16392)):
        say("reg tile", block, M, N)
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        x[M // 2] = 0
        q, s = fq.quantize(x, block)
        assert_matches_oracle(x, q, s, bm, bn, f"reg {M}x{N}/{block}")
    outs = fq.quantize_many([x, x[:100].contiguous()], block)
    assert torch.equal(outs[0][0].view(torch.uint8), q.view(torch.uint8))


def test_special_values(gpu_lib):
    """Zero, -0, BF16 subnormals, huge magnitudes and exact e4m3 ties."""
    rows = []
    ties = [448.0, 1.0625, -1.1875, 0.0029296875, 248.0, -400.0, 432.0, 2.0 ** -10]
    rows.append(np.array(ties + [0.0] * 120, dtype=np.float32))
    rows.append(np.array([-0.0] * 128, dtype=np.float32))
    rows.append(np.zeros(128, dtype=np.float32))
    sub = np.array([((i % 127) + 1) * 2.0 ** -133 for i in range(128)], dtype=np.float32)
    rows.append(sub * np.where(np.arange(128) % 2, -1, 1))
    rows.append(np.linspace(-3.3e38, 3.3e38, 128).astype(np.float32))
    rows.append(np.array([1e-12] * 64 + [-3e-11] * 64, dtype=np.float32))  # below eps
    x32 = torch.from_numpy(np.stack(rows))
    x = x32.to(torch.bfloat16).to(DEV)
    for bm, bn in [(1, 128), (128, 128), (64, 64), (2, 3), (6, 128)]:
        q, s = fq.quantize(x, (bm, bn))
        assert_matches_oracle(x, q, s, bm, bn, f"special/{bm}x{bn}")


# ------------------------------------------------------------------ sweeps

def _anchor_rows(anchors, rng):
    """[1,128] rows: column 0 holds the anchor, the rest sweep every BF16
    magnitude at or below it (random signs)."""
    rows = []
    for a in anchors:
        mags = np.arange(0, a + 1, dtype=np.uint32)
        mags = mags[rng.permutation(mags.size)]
        pad = (-mags.size) % 127
        mags = np.concatenate([mags, np.zeros(pad, dtype=np.uint32)]).reshape(-1, 127)
        sign = (rng.integers(0, 2, mags.shape).astype(np.uint32) << 15)
        body = (mags | sign).astype(np.uint16)
        anchor = np.full((body.shape[0], 1), a, dtype=np.uint16)
        anchor |= (rng.integers(0, 2, anchor.shape).astype(np.uint16) << 15)
        rows.append(np.concatenate([anchor, body], axis=1))
    return np.concatenate(rows)


def test_anchor_sweep_every_bf16(gpu_lib):
    """Every finite BF16 magnitude below each of many anchors, through the
    [1,128] kernel and (re-tiled) the [128,128] kernel."""
    rng = np.random.default_rng(2024)
    anchors = sorted(set(int(v) for v in rng.integers(0x0080, 0x7F7F, 120)) |
                     {0x43E0, 0x3F80, 0x40A0, 0x7F7F, 0x0001, 0x2EDB, 0x2EDC})
    for i in range(0, len(anchors), 16):
        bits = _anchor_rows(anchors[i:i + 16], rng)
        x = bf16_from_bits(bits)
        say("anchors", i, bits.shape)
        q, s = fq.quantize(x, (1, 128))
        assert_matches_oracle(x, q, s, 1, 128, f"anchor rows {i}")
        rows = (bits.shape[0] // 128) * 128
        if rows:
            xt = x[:rows].contiguous()
            for block in [(128, 128), (64, 64), (32, 128), (7, 64)]:
                q, s = fq.quantize(xt, block)
                assert_matches_oracle(xt, q, s, *block, f"anchor tiles {i} {block}")


def _double_rounding_rows(min_rows=256):
    """[1,128] rows: an anchor maximum in column 0 and BF16 values whose
    scaled product x*r rounds (in float32) exactly onto an e4m3 midpoint
    without being on it, so the float32 rounding decides the code."""
    rng = np.random.default_rng(67)
    pos = np.array([float(v) for v in oracle.e4m3fn.decode_np(np.arange(127, dtype=np.uint8))])
    mids = (pos[:-1] + pos[1:]) / 2
    rows = []
    while len(rows) < min_rows:
        ab = int(rng.integers(0x2000, 0x6000))
        a = float(oracle.bf16_bits_to_f64([ab])[0])
        _, r = oracle.tile_scale(a)
        xb = np.arange(1, ab, dtype=np.uint16)
        p = oracle.bf16_bits_to_f64(xb) * r
        y = p.astype(np.float32).astype(np.float64)
        hit = xb[np.isin(y, mids) & (p != y)]
        for i in range(0, hit.size, 63):
            h = hit[i:i + 63]
            row = np.zeros(128, dtype=np.uint16)
            row[0] = ab
            row[1:1 + h.size] = h
            row[64:64 + h.size] = h | 0x8000
            rows.append(row)
    return np.stack(rows)


def test_double_rounding_cases_all_kinds(gpu_lib):
    """Inputs where the float32 rounding of x*r decides the e4m3 code, through
    every kernel body: [1,128] rows, [128,128] and [64,64] tiles (re-tiled),
    the register tile body and the element-wise body."""
    bits = _double_rounding_rows()
    rows = (bits.shape[0] // 128) * 128
    assert rows >= 128, "the search found too few cases"
    x = bf16_from_bits(bits[:rows])
    say("double rounding rows", rows)
    for block in [(1, 128), (128, 128), (64, 64), (16, 128), (3, 5)]:
        q, s = fq.quantize(x, block)
        assert_matches_oracle(x, q, s, *block, f"double rounding {block}")


def test_encoder_exhaustive_fp32(gpu_lib):
    """The hardware convert over every float32 from 0 to 448 (and negatives,
    and everything above 448 after the clamp): equal to the oracle encoder.

    The codes of the positive patterns form a non-decreasing step function of
    the bit pattern; so does the oracle's (a composition of monotone steps),
    so agreement at both sides of every GPU step edge plus a strided sample
    proves agreement everywhere."""
    top = 0x43E00000  # 448.0
    chunk = 1 << 27
    prev_last = None
    checked = 0
    for start in range(0, top + 1, chunk):
        end = min(top + 1, start + chunk)
        pat = torch.arange(start, end, dtype=torch.int32, device=DEV)
        y = pat.view(torch.float32)
        c = fq.encode_e4m3(y)
        cn = fq.encode_e4m3((pat | torch.tensor(-0x80000000, dtype=torch.int32, device=DEV))
                            .view(torch.float32))
        assert torch.equal(cn, c | 0x80), ("negative", start)
        assert bool((c[1:] >= c[:-1]).all()), ("monotone", start)
        if prev_last is not None:
            assert int(c[0]) >= prev_last
        prev_last = int(c[-1])
        edges = torch.nonzero(c[1:] != c[:-1]).flatten().cpu().numpy()
        idx = np.unique(np.concatenate([edges, edges + 1, [0, end - start - 1],
                                        np.arange(0, end - start, 4099)]))
        got = c.cpu().numpy()[idx]
        vals = (idx.astype(np.int64) + start).astype(np.uint32).view(np.float32).astype(np.float64)
        want = oracle.encode_np(vals)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(float(vals[i]), int(got[i]), int(want[i])) for i in bad[:5]]
        checked += idx.size
        say("encoder chunk", hex(start), "edges", edges.size)
    assert checked > 0
    # above 448: the clamp sends every finite value to 0x7E / 0xFE
    for start in range(top + 1, 0x7F800000, chunk):
        end = min(0x7F800000, start + chunk)
        pat = torch.arange(start, end, dtype=torch.int32, device=DEV)
        assert bool((fq.encode_e4m3(pat.view(torch.float32)) == 0x7E).all())
        neg = (pat | torch.tensor(-0x80000000, dtype=torch.int32, device=DEV)).view(torch.float32)
        assert bool((fq.encode_e4m3(neg) == 0xFE).all())


# ------------------------------------------------------------------ weight sets

def test_c2_layer_grouped_equals_oracle_and_single(gpu_lib):
    specs = wl.c2()
    xs = [wl.materialize(sp, DEV) for sp in specs]
    outs = fq.quantize_many(xs, (128, 128))
    torch.cuda.synchronize()
    for sp, x, (q, s) in zip(specs, xs, outs):
        say("C2", sp.name)
        assert_matches_oracle(x, q, s, 128, 128, sp.name)
        q1, s1 = fq.quantize(x, (128, 128))
        assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8))
        assert torch.equal(s1.view(torch.int32), s.view(torch.int32))


def test_determinism_and_canaries(gpu_lib):
    """Same bytes on every run; nothing written outside q and scale_inv."""
    G = 256
    g = torch.Generator(device=DEV).manual_seed(5)
    for M, N, block in ((77, 128, (128, 128)), (4097, 11008, (128, 128)), (1000, 3000, (64, 64)),
                        (1000, 3000, (1, 128)), (129, 1001, (128, 128)), (33, 40, (5, 7))):
        say("canary", M, N, block)
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
        TM, TN = fq.scale_shape(M, N, *block)
        results = []
        for _ in range(2):
            qb = torch.full((M * N + 2 * G,), 0xA5, dtype=torch.uint8, device=DEV)
            sb = torch.full((TM * TN + 2 * G,), -7.5, dtype=torch.float32, device=DEV)
            q = qb[G:G + M * N].view(M, N)
            s = sb[G:G + TM * TN].view(TM, TN)
            fq.quantize(x, block, out=(q, s))
            torch.cuda.synchronize()
            assert bool((qb[:G] == 0xA5).all()) and bool((qb[G + M * N:] == 0xA5).all())
            assert bool((sb[:G] == -7.5).all()) and bool((sb[G + TM * TN:] == -7.5).all())
            results.append((q.clone(), s.clone()))
        assert torch.equal(results[0][0], results[1][0])
        assert torch.equal(results[0][1].view(torch.int32), results[1][1].view(torch.int32))


def test_non_finite_input_stays_in_bounds(gpu_lib):
    """NaN and Inf are outside the contract: their tiles' outputs are
    unspecified, but every write stays inside q and scale_inv and finite
    tiles are unaffected."""
    G = 256
    g = torch.Generator(device=DEV).manual_seed(71)
    for M, N, block in ((300, 520, (128, 128)), (300, 520, (64, 64)), (300, 520, (1, 128)),
                        (300, 520, (16, 64)), (301, 519, (128, 128)), (300, 520, (300, 520))):
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        x[5, 7] = float("nan")
        x[200, 300] = float("inf")
        x[250, 10] = float("-inf")
        TM, TN = fq.scale_shape(M, N, *block)
        qb = torch.full((M * N + 2 * G,), 0xA5, dtype=torch.uint8, device=DEV)
        sb = torch.full((TM * TN + 2 * G,), -7.5, dtype=torch.float32, device=DEV)
        q, s = qb[G:G + M * N].view(M, N), sb[G:G + TM * TN].view(TM, TN)
        fq.quantize(x, block, out=(q, s))
        torch.cuda.synchronize()
        assert bool((qb[:G] == 0xA5).all()) and bool((qb[G + M * N:] == 0xA5).all()), block
        assert bool((sb[:G] == -7.5).all()) and bool((sb[G + TM * TN:] == -7.5).all()), block
        # tiles without a non-finite value match a finite copy quantized alone
        xf = torch.nan_to_num(x.float(), nan=0.0, posinf=0.0, neginf=0.0).to(torch.bfloat16)
        q2, s2 = fq.quantize(xf, block)
        bad_rows = {5 // block[0], 200 // block[0], 250 // block[0]}
        bad = {(5 // block[0], 7 // block[1]), (200 // block[0], 300 // block[1]),
               (250 // block[0], 10 // block[1])}
        for ti in range(TM):
            for tj in range(TN):
                if (ti, tj) in bad:
                    continue
                r0, c0 = ti * block[0], tj * block[1]
                assert torch.equal(q[r0:r0 + block[0], c0:c0 + block[1]],
                                   q2.view(torch.uint8)[r0:r0 + block[0], c0:c0 + block[1]]), (block, ti, tj)
        assert bad_rows


def test_grouped_mixed_list(gpu_lib):
    """One grouped launch over empty, odd-N, misaligned and aligned tensors
    equals single calls and the oracle, for every block kind."""
    g = torch.Generator(device=DEV).manual_seed(11)
    base = (torch.randn(600 * 1001 + 16, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    mats = [
        (torch.randn((300, 512), generator=g, device=DEV) * 0.02).to(torch.bfloat16),
        torch.empty((0, 128), dtype=torch.bfloat16, device=DEV),
        base[1:1 + 129 * 1001].view(129, 1001),                       # odd N, misaligned
        (torch.randn((1, 8), generator=g, device=DEV)).to(torch.bfloat16),
        torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV),
        base[8:8 + 200 * 136].view(200, 136),                          # aligned view
        torch.empty((5, 0), dtype=torch.bfloat16, device=DEV),
        (torch.randn((1537, 2048), generator=g, device=DEV) * 0.03).to(torch.bfloat16),
    ]
    for block in BLOCKS + [(3, 5), (1024, 1024)]:   # the last: large tiles, grouped two-pass kernels
        say("mixed", block)
        outs = fq.quantize_many(mats, block)
        for i, (x, (q, s)) in enumerate(zip(mats, outs)):
            if x.numel() == 0:
                continue
            assert_matches_oracle(x, q, s, *block, f"mixed[{i}]/{block}")
            q1, s1 = fq.quantize(x, block)
            assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8))


def test_grouped_workspace_path(gpu_lib, oracle_pool):
    """More than 512 tensors: the descriptor table goes through the workspace
    (host-to-device copy) instead of the kernel arguments."""
    g = torch.Generator(device=DEV).manual_seed(13)
    rng = np.random.default_rng(13)
    mats = []
    for _ in range(700):
        M, N = int(rng.integers(1, 300)), int(rng.choice([8, 64, 136, 256, 264, 7, 99]))
        mats.append((torch.randn((M, N), generator=g, device=DEV) * 0.03).to(torch.bfloat16))
    assert fq.workspace_bytes(len(mats)) > 0
    # (300, 300): tensors with more than 65536 elements per tile take the
    # grouped two-pass kernels, the rest the workspace path, in one call
    for block in BLOCKS + [(5, 3), (300, 300)]:
        say("workspace path", block)
        outs = fq.quantize_many(mats, block)
        for i, (x, (q, s)) in enumerate(zip(mats, outs)):
            q1, s1 = fq.quantize(x, block)
            assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), (block, i)
            assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), (block, i)
        chk = FullOracleCheck(oracle_pool, *block, f"workspace path {block}")
        for i, (x, (q, s)) in enumerate(zip(mats, outs)):
            chk.add(f"[{i}]", x, q, s)
        chk.finish()


@pytest.mark.parametrize("bm,bn", BLOCKS)
def test_c5_ragged_full(gpu_lib, oracle_pool, bm, bn):
    """The ragged set (1000x3000, 4097x11008, 151937x4096, 77x128) at each
    block size, one single call per matrix: every byte and scale against
    the oracle, plus the invariants."""
    chk = FullOracleCheck(oracle_pool, bm, bn, f"C5 [{bm},{bn}]")
    for sp in wl.c5():
        x = wl.materialize(sp, DEV)
        q, s = fq.quantize(x, (bm, bn))
        say("C5", sp.name, bm, bn)
        assert_properties_gpu(x, q, s, bm, bn, sp.name)
        chk.add(sp.name, x, q, s)
        del x, q, s
    n, values = chk.finish()
    say("C5 compared whole:", n, "matrices,", values, "values")


def test_c3_dense_stack_one_grouped_launch(gpu_lib, oracle_pool):
    """The 36-layer dense weight set (252 tensors, 13.9 GB) in the one grouped
    launch the benchmark times: every byte and every scale of all 252
    outputs against the oracle, plus the invariants."""
    specs = wl.c3()
    xs = [wl.materialize(sp, DEV) for sp in specs]
    say("C3 generated", len(xs))
    outs = fq.quantize_many(xs, (128, 128))
    torch.cuda.synchronize()
    chk = FullOracleCheck(oracle_pool, 128, 128, "C3")
    for sp, x, (q, s) in zip(specs, xs, outs):
        assert_properties_gpu(x, q, s, 128, 128, sp.name)
        chk.add(sp.name, x, q, s)
    n, values = chk.finish()
    assert (n, values) == (252, 6_945_767_424)
    say("C3 compared whole:", n, "tensors,", values, "values")


@pytest.mark.parametrize("block", [(128, 128), (64, 64)])
def test_wide_unit_launch(gpu_lib, oracle_pool, block):
    """A [128,128] or [64,64] launch that takes the wide unit (128x512: four
    tiles; 64x512: eight): widths that are multiples of 512 and at least 8192
    such units in all (a 1 GB matrix whose last unit row is partial), grouped
    with a misaligned tensor (a general body in the same launch), a
    ragged-height tensor and an empty one.  The large matrix is compared with
    the oracle whole, every byte and scale; the small tensors equal their
    single calls (narrow units)."""
    bm, bn = block
    g = torch.Generator(device=DEV).manual_seed(61)
    big = (torch.randn((32768 - 56, 16384), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    flat = (torch.randn(1000 * 4096 + 1, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    mis = flat[1:].view(1000, 4096)                   # 2 bytes past a 16-byte boundary
    ragged = (torch.randn((777, 1024), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    xs = [ragged, big, mis, empty]
    say("wide-unit launch", block)
    outs = fq.quantize_many(xs, block)
    torch.cuda.synchronize()
    assert_properties_gpu(big, outs[1][0], outs[1][1], bm, bn, "wide big")
    chk = FullOracleCheck(oracle_pool, bm, bn, f"wide launch {block}")
    chk.add("wide big", big, *outs[1])
    chk.finish()
    for x, (q, s), name in ((ragged, outs[0], "ragged"), (mis, outs[2], "misaligned")):
        q1, s1 = fq.quantize(x, block)
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), name
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), name
    assert_matches_oracle(ragged, outs[0][0], outs[0][1], bm, bn, "ragged in wide launch")
    del big, outs


@pytest.mark.parametrize("part", range(4))
def test_c4_moe_per_layer_grouped(gpu_lib, oracle_pool, part):
    """MoE weight set: 48 layers x 256 expert matrices, one grouped launch per
    layer (12 layers per test): every byte and every scale of every expert
    matrix against the oracle, and the per-tile maximum code on the GPU."""
    chk = FullOracleCheck(oracle_pool, 128, 128, f"C4 layers {part * 12}..{part * 12 + 11}")
    for layer in range(part * 12, part * 12 + 12):
        specs = wl.c4_layer(layer)
        xs = [wl.materialize(sp, DEV) for sp in specs]
        outs = fq.quantize_many(xs, (128, 128))
        say("C4 layer", layer)
        for j in (0, 1):
            sub = list(range(j, len(xs), 2))
            E, M, N = len(sub), *xs[j].shape
            qg = torch.stack([outs[k][0].view(torch.uint8) for k in sub])
            assert not bool(((qg == 0x7F) | (qg == 0xFF)).any())
            tmax = (qg & 0x7F).view(E, M // 128, 128, N // 128, 128).amax(dim=(2, 4))
            assert bool((tmax == 0x7E).all()), layer
            del qg
        for sp, x, (q, s) in zip(specs, xs, outs):
            chk.add(sp.name, x, q, s)
        del xs, outs
    n, values = chk.finish()
    assert n == 12 * 256
    say("C4 compared whole:", n, "matrices,", values, "values")


# ------------------------------------------------------------------ dequantization

@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_dequant_matches_oracle(gpu_lib, out_dtype):
    """decode(q) * s on the GPU equals the oracle, bit for bit, on the vector
    kernel (N % 16 == 0, bn % 16 == 0, aligned) and the element-wise kernel."""
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=DEV).manual_seed(31)
    cases = [(256, 256, (128, 128)), (1000, 3000, (64, 64)), (77, 128, (1, 128)),
             (4097, 1008, (128, 128)), (129, 1001, (128, 128)), (300, 520, (3, 5)),
             (65, 48, (16, 16)), (33, 40, (1, 1))]
    for M, N, block in cases:
        say("dequant", out_dtype, M, N, block)
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
        x[0] = 0
        q, s = fq.quantize(x, block)
        xh = fq.dequantize(q, s, block, out_dtype=tdt)
        torch.cuda.synchronize()
        want = oracle.dequantize(codes_np(q), s.cpu().numpy(), *block, out_dtype)
        got = xh.float().cpu().numpy().astype(np.float64)
        bad = np.nonzero(got != want)
        assert bad[0].size == 0, (M, N, block, bad[0].size)
        # misaligned q and out take the element-wise kernel
        qb = torch.empty(M * N + 16, dtype=torch.uint8, device=DEV)
        q2 = qb[1:1 + M * N].view(M, N)
        q2.copy_(q.view(torch.uint8))
        ob = torch.empty(M * N + 8, dtype=tdt, device=DEV)
        o2 = ob[1:1 + M * N].view(M, N)
        fq.dequantize(q2, s, block, out_dtype=tdt, out=o2)
        assert torch.equal(o2.float(), xh.float())


def test_dequant_seeded_fuzz(gpu_lib):
    """120 seeded random dequantizations (random codes without NaN, random
    positive scales per tile over 2^-30..2^30) against the oracle, fp32 and
    BF16: shapes up to 700 x 1600, N and bn multiples of 8 in most cases
    (the vector kernel, whose row, tile-row and tile-column indices come from
    multiply-and-shift divisions) and arbitrary otherwise."""
    rng = np.random.default_rng(4242)
    for i in range(120):
        out_dtype = "f32" if i % 2 == 0 else "bf16"
        tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        vec = rng.random() < 0.75
        M = int(rng.integers(1, 701))
        N = int(rng.integers(1, 201)) * 8 if vec else int(rng.integers(1, 1601))
        bm = int(rng.integers(1, 301))
        bn = int(rng.integers(1, 41)) * 8 if vec else int(rng.integers(1, 301))
        TM, TN = -(-M // bm), -(-N // bn)
        codes = rng.integers(0, 256, (M, N), dtype=np.int64).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] ^= 0x01                  # no NaN codes
        scales = np.exp2(rng.uniform(-30, 30, (TM, TN))).astype(np.float32)
        q = torch.from_numpy(codes).to(DEV)
        s = torch.from_numpy(scales).to(DEV)
        say("dequant fuzz", i, M, N, (bm, bn), out_dtype)
        xh = fq.dequantize(q, s, (bm, bn), out_dtype=tdt)
        want = oracle.dequantize(codes, scales, bm, bn, out_dtype)
        got = xh.float().cpu().numpy().astype(np.float64)
        bad = np.nonzero(got != want)
        assert bad[0].size == 0, (i, M, N, bm, bn, out_dtype, bad[0].size)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_many_matches_single_calls(gpu_lib, out_dtype):
    """Grouped dequantization of 300 entries (two launches of up to 256),
    mixing vector-kernel entries with ragged shapes, entries that take the
    element-wise kernel (N % 8 != 0, an output 4 bytes past a 16-byte
    boundary) and empty ones: every output equals its single call bit for
    bit, and seeded entries equal the oracle."""
    rng = np.random.default_rng(909)
    bm, bn = 64, 128
    qs, ss, outs, codes_l, scales_l = [], [], [], [], []
    esize = 4 if out_dtype == torch.float32 else 2
    for i in range(300):
        kind = i % 10
        M = 0 if kind == 9 else int(rng.integers(1, 300))
        N = int(rng.integers(1, 300)) if kind == 7 else int(rng.integers(1, 40)) * 8
        TM, TN = -(-max(M, 1) // bm), -(-N // bn)
        codes = rng.integers(0, 256, (M, N), dtype=np.int64).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] ^= 0x01
        scales = np.exp2(rng.uniform(-20, 20, (-(-M // bm), TN))).astype(np.float32)
        qs.append(torch.from_numpy(codes).to(DEV))
        ss.append(torch.from_numpy(scales).to(DEV))
        if kind == 8 and M > 0:                      # output 4 bytes past a 16-byte boundary
            buf = torch.empty(M * N * esize + 16, dtype=torch.uint8, device=DEV)
            outs.append(buf[4:4 + M * N * esize].view(out_dtype).view(M, N))
        else:
            outs.append(torch.empty((M, N), dtype=out_dtype, device=DEV))
        codes_l.append(codes)
        scales_l.append(scales)
    say("dequantize_many", out_dtype)
    got = fq.dequantize_many(qs, ss, (bm, bn), out_dtype=out_dtype, outs=outs)
    torch.cuda.synchronize()
    for i, (q, s, o) in enumerate(zip(qs, ss, got)):
        if q.numel() == 0:
            continue
        one = fq.dequantize(q, s, (bm, bn), out_dtype=out_dtype)
        assert torch.equal(o.view(torch.int16 if esize == 2 else torch.int32),
                           one.view(torch.int16 if esize == 2 else torch.int32)), i
    # a short list (one block per unit for either output type)
    few = fq.dequantize_many(qs[:6], ss[:6], (bm, bn), out_dtype=out_dtype)
    for i, o in enumerate(few):
        if qs[i].numel():
            assert torch.equal(o.view(torch.uint8), got[i].contiguous().view(torch.uint8)), i
    name = "f32" if out_dtype == torch.float32 else "bf16"
    for i in range(len(codes_l)):
        if codes_l[i].size == 0:
            continue
        want = oracle.dequantize(codes_l[i], scales_l[i], bm, bn, name)
        assert np.array_equal(got[i].float().cpu().numpy().astype(np.float64), want), i


def test_dequant_roundtrip_bound_layer(gpu_lib):
    """I4 over a whole Qwen3-8B-shaped layer on the GPU: |x - dequant(q)| is
    within half an e4m3 ulp of the scaled value times s (+ fp32 rounding)."""
    for sp in wl.c2():
        x = wl.materialize(sp, DEV)
        q, s = fq.quantize(x, (128, 128))
        xh = fq.dequantize(q, s, (128, 128)).double()
        xd = x.double()
        sf = s.double().repeat_interleave(128, 0)[:sp.M].repeat_interleave(128, 1)[:, :sp.N]
        y = xd.abs() / sf
        e = torch.floor(torch.log2(torch.clamp(y, min=2.0 ** -6)))
        ulp = torch.where(y >= 2.0 ** -6, torch.exp2(e - 3), torch.full_like(y, 2.0 ** -9))
        ok = (xd - xh).abs() <= 0.5 * ulp * sf + 2.0 ** -21 * xd.abs()
        assert bool(ok.all()), sp.name
        del x, q, s, xh, xd, sf, y, e, ulp, ok


# ------------------------------------------------------------------ large tiles and shards

def _shards(x, block, row_cuts, col_cuts):
    """Quantize ``x`` shard by shard on the GPU: partial maxima per shard,
    an element-wise max over shards sharing a tile (the exchange), then
    each shard quantized with the full maxima; returns assembled (q, s)."""
    bm, bn = block
    M, N = x.shape
    TM, TN = fq.scale_shape(M, N, bm, bn)
    full = torch.zeros((TM, TN), dtype=torch.float32, device=DEV)
    rb, cb = [0] + row_cuts + [M], [0] + col_cuts + [N]
    parts = []
    for i in range(len(rb) - 1):
        for j in range(len(cb) - 1):
            r0, r1, c0, c1 = rb[i], rb[i + 1], cb[j], cb[j + 1]
            if r0 == r1 or c0 == c1:
                continue
            xs = x[r0:r1, c0:c1].contiguous()
            ph = (r0 % bm, c0 % bn)
            a = fq.tile_amax(xs, block, ph)
            t0, u0 = r0 // bm, c0 // bn
            v = full[t0:t0 + a.shape[0], u0:u0 + a.shape[1]]
            v.copy_(torch.maximum(v, a))
            parts.append((r0, r1, c0, c1, xs, ph, t0, u0, a.shape))
    q = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    s = torch.empty((TM, TN), dtype=torch.float32, device=DEV)
    for r0, r1, c0, c1, xs, ph, t0, u0, shp in parts:
        am = full[t0:t0 + shp[0], u0:u0 + shp[1]].contiguous()
        qs, ss = fq.quantize_with_amax(xs, am, block, ph)
        q[r0:r1, c0:c1] = qs.view(torch.uint8)
        s[t0:t0 + shp[0], u0:u0 + shp[1]] = ss
    return q, s


def test_tile_amax_and_quantize_amax_match_oracle(gpu_lib):
    g = torch.Generator(device=DEV).manual_seed(41)
    rng = np.random.default_rng(41)
    for M, N, block in [(300, 520, (128, 128)), (77, 200, (64, 64)), (129, 257, (1, 128)),
                        (50, 61, (7, 9)), (1000, 3000, (512, 512)), (64, 100000, (1, 100000))]:
        bm, bn = block
        for _ in range(3):
            ph = (int(rng.integers(bm)), int(rng.integers(bn)))
            say("amax", M, N, block, ph)
            x = (torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
            a = fq.tile_amax(x, block, ph)
            xb = bits_np(x)
            a_ref = oracle.tile_amax(xb, bm, bn, *ph)
            assert np.array_equal(a.cpu().numpy().astype(np.float64), a_ref)
            q, s = fq.quantize_with_amax(x, a, block, ph)
            q_ref, s_ref = oracle.quantize_with_amax(xb, bm, bn, a_ref, *ph)
            assert np.array_equal(codes_np(q), q_ref)
            assert np.array_equal(scales_bits(s), scales_bits(s_ref))


def test_shard_small_tile_kernels(gpu_lib):
    """Shards whose tiles hold at most 16,384 elements and whose tile columns
    start on 8-element boundaries (one workgroup per tile, or 64 one-row
    tiles per workgroup for [1, <=128] blocks: maxima stored directly,
    quantize and scales in one launch), at random row phases and 8-aligned
    column phases; also with the maxima converted in place (amax passed as
    scale_inv)."""
    g = torch.Generator(device=DEV).manual_seed(47)
    rng = np.random.default_rng(47)
    for M, N, block in [(300, 520, (128, 128)), (1000, 3000, (64, 64)), (257, 384, (32, 128)),
                        (129, 256, (1, 128)), (50, 64, (8, 8)), (2000, 1024, (128, 64)),
                        (3, 4096, (2, 4096)), (127, 8, (127, 8)), (300, 1000, (1, 64)),
                        (17, 40, (1, 8)), (70, 1024, (1, 120))]:
        bm, bn = block
        for _ in range(3):
            ph = (int(rng.integers(bm)), 8 * int(rng.integers(bn // 8)))
            say("small-tile shard", M, N, block, ph)
            x = (torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
            xb = bits_np(x)
            a = fq.tile_amax(x, block, ph)
            a_ref = oracle.tile_amax(xb, bm, bn, *ph)
            assert np.array_equal(a.cpu().numpy().astype(np.float64), a_ref), (M, N, block, ph)
            q, s = fq.quantize_with_amax(x, a, block, ph)
            q_ref, s_ref = oracle.quantize_with_amax(xb, bm, bn, a_ref, *ph)
            assert np.array_equal(codes_np(q), q_ref), (M, N, block, ph)
            assert np.array_equal(scales_bits(s), scales_bits(s_ref)), (M, N, block, ph)
            a2 = a.clone()
            q2 = torch.empty_like(q)
            fq.quantize_with_amax(x, a2, block, ph, out=(q2, a2))    # maxima -> scales in place
            assert torch.equal(q2.view(torch.uint8), q.view(torch.uint8))
            assert torch.equal(a2.view(torch.int32), s.view(torch.int32))


def test_shard_many_four_tile_units(gpu_lib):
    """The grouped [128,128] quantize pass takes four-tile units where four
    whole tiles lie inside a shard and single tiles elsewhere: wide shards at
    row and column phases (whole and partial units, widths not a multiple of
    512) equal the single calls, also with the maxima converted in place,
    and every maximum, code and scale equals the oracle's."""
    g = torch.Generator(device=DEV).manual_seed(67)
    xs, phases = [], []
    for i, (M, N, ph) in enumerate([(1000, 2048, (64, 0)), (1000, 2048, (0, 64)), (777, 1536, (0, 0)),
                                    (300, 4096, (127, 8)), (129, 640, (1, 0)), (2048, 1000, (0, 0))] * 4):
        xs.append((torch.randn((M, N), generator=g, device=DEV) * (0.01 + 0.01 * i)).to(torch.bfloat16))
        phases.append(ph)
    amaxs = fq.tile_amax_many(xs, (128, 128), phases)
    outs = fq.quantize_with_amax_many(xs, amaxs, (128, 128), phases)
    # maxima converted to scales in place: the table's scale_inv is amax itself
    inplace = [a.clone() for a in amaxs]
    q2s = [torch.empty_like(q) for q, _ in outs]
    table = fq._shard_table(xs, phases, q2s, inplace, inplace)
    lib = fq.load_library()
    assert lib.fp8bq_quantize_amax_many(table, len(xs), 128, 128,
                                        torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    outs2 = list(zip(q2s, inplace))
    for i, (x, ph, a, (q, s), (q2, s2)) in enumerate(zip(xs, phases, amaxs, outs, outs2)):
        q1, s1 = fq.quantize_with_amax(x, a, (128, 128), ph)
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), i
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), i
        assert torch.equal(q2.view(torch.uint8), q1.view(torch.uint8)), i
        assert torch.equal(s2.view(torch.int32), s1.view(torch.int32)), i
    for i in range(len(xs)):
        xb = bits_np(xs[i])
        a_ref = oracle.tile_amax(xb, 128, 128, *phases[i])
        assert np.array_equal(amaxs[i].double().cpu().numpy(), a_ref), i
        q_ref, s_ref = oracle.quantize_with_amax(xb, 128, 128, a_ref, *phases[i])
        assert np.array_equal(codes_np(outs[i][0]), q_ref), i
        assert np.array_equal(scales_bits(outs[i][1]), scales_bits(s_ref)), i


@pytest.mark.parametrize("block", [(128, 128), (64, 64), (1, 128), (32, 96)])
def test_shard_many_matches_single_calls(gpu_lib, block):
    """Grouped shard calls over 600 shards (more than one 512-entry launch)
    mixing small aligned tiles with entries that take their own launches
    (N % 8 != 0, a misaligned x, odd column phases) and empty shards: every
    maximum, code and scale equals the single calls' and the oracle's; maxima
    converted in place (amax passed as scale_inv) give the same scales."""
    import ctypes

    bm, bn = block
    g = torch.Generator(device=DEV).manual_seed(53)
    rng = np.random.default_rng(53)
    xs, phases = [], []
    for i in range(600):
        M = int(rng.integers(0 if i % 97 == 0 else 1, 300))
        N = int(rng.choice([8, 64, 128, 136, 256, 520, 77]))
        cp = 8 * int(rng.integers(max(1, bn // 8))) if i % 5 else int(rng.integers(bn))
        ph = (int(rng.integers(bm)), min(cp, bn - 1))
        flat = (torch.randn(M * N + 1, generator=g, device=DEV) * 0.03).to(torch.bfloat16)
        # every 11th shard starts 2 bytes past a 16-byte boundary (contiguous view)
        xs.append(flat[1:].view(M, N) if i % 11 == 0 else flat[:-1].view(M, N))
        phases.append(ph)
    say("shard many", block, len(xs))
    amaxs = fq.tile_amax_many(xs, block, phases)
    outs = fq.quantize_with_amax_many(xs, amaxs, block, phases)
    for i, (x, ph, a, (q, s)) in enumerate(zip(xs, phases, amaxs, outs)):
        if x.numel() == 0:
            continue                          # an empty shard writes nothing
        a1 = fq.tile_amax(x, block, ph)
        assert torch.equal(a.view(torch.int32), a1.view(torch.int32)), (block, i)
        q1, s1 = fq.quantize_with_amax(x, a1, block, ph)
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), (block, i)
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), (block, i)
    for i in range(len(xs)):
        xb = bits_np(xs[i])
        if xb.size == 0:
            continue
        a_ref = oracle.tile_amax(xb, bm, bn, *phases[i])
        q_ref, s_ref = oracle.quantize_with_amax(xb, bm, bn, a_ref, *phases[i])
        assert np.array_equal(codes_np(outs[i][0]), q_ref) and np.array_equal(
            scales_bits(outs[i][1]), scales_bits(s_ref)), (block, i)
    # in place: scale_inv is amax itself, through the C ABI
    inplace = [a.clone() for a in amaxs]
    qs = [torch.empty_like(q) for q, _ in outs]
    arr = (fq.ShardEntry * len(xs))()
    for e, x, ph, a, q in zip(arr, xs, phases, inplace, qs):
        e.x, e.q, e.amax, e.scale_inv = x.data_ptr(), q.data_ptr(), a.data_ptr(), a.data_ptr()
        e.M, e.N = x.shape
        e.row_phase, e.col_phase = ph
    st = gpu_lib.load_library().fp8bq_quantize_amax_many(
        arr, len(xs), bm, bn, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for i, (x, a, q, (q1, s1)) in enumerate(zip(xs, inplace, qs, outs)):
        if x.numel() == 0:
            continue
        assert torch.equal(a.view(torch.int32), s1.view(torch.int32)), (block, i)
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), (block, i)


def test_shards_equal_whole(gpu_lib):
    """Cuts anywhere (inside tiles too): shard-wise maxima, exchanged as a
    max, then shard-wise quantization reproduce the whole-matrix bytes."""
    g = torch.Generator(device=DEV).manual_seed(43)
    rng = np.random.default_rng(43)
    # the last two: large tiles whose maxima pass groups several chunks per
    # workgroup (one tile per tensor: 4 chunks per item; 1024 x 2000 tiles)
    for M, N, block in [(1000, 3000, (128, 128)), (4097, 1024, (64, 64)), (300, 640, (1, 128)),
                        (1536, 2048, (128, 128)), (4096, 4096, (4096, 4096)),
                        (3000, 2000, (1024, 2000))]:
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        q_ref, s_ref = fq.quantize(x, block)
        a = fq.tile_amax(x, block)                          # whole matrix, phase (0, 0)
        assert np.array_equal(a.cpu().numpy().astype(np.float64), tile_amax_gpu(x, *block))
        for _ in range(4):
            rc = sorted(set(int(v) for v in rng.integers(1, M, rng.integers(1, 5))))
            cc = sorted(set(int(v) for v in rng.integers(1, N, rng.integers(0, 3))))
            say("shards", M, N, block, rc, cc)
            q, s = _shards(x, block, rc, cc)
            assert torch.equal(q, q_ref.view(torch.uint8)), (rc, cc)
            assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32)), (rc, cc)


def test_per_tensor_and_large_tiles(gpu_lib):
    """Tiles above 65536 elements (one scale per tensor, wide rows, big
    squares) through fp8bq_quantize and the grouped call."""
    g = torch.Generator(device=DEV).manual_seed(47)
    for M, N, block in [(1000, 3000, (1000, 3000)), (4097, 1008, (4097, 1008)),
                        (300, 520, (512, 512)), (33, 70001, (1, 70001)), (129, 1001, (129, 1001)),
                        (1536, 2048, (1024, 1024))]:
        say("large", M, N, block)
        x = (torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
        x[0] = 0
        q, s = fq.quantize(x, block)
        assert_matches_oracle(x, q, s, *block, f"large {M}x{N}/{block}")
    # misaligned x / odd N take the scalar paths of the same kernels
    big = (torch.randn(999 * 1001 + 8, generator=g, device=DEV)).to(torch.bfloat16)
    x = big[3:3 + 999 * 1001].view(999, 1001)
    q, s = fq.quantize(x, (999, 1001))
    assert_matches_oracle(x, q, s, 999, 1001, "large misaligned")
    # q at odd byte addresses (pass 1 keeps its partial maxima in q from the
    # first 4-byte boundary): same bytes, nothing written outside q
    x = (torch.randn((700, 1200), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    q0, s0 = fq.quantize(x, (700, 1200))
    assert_matches_oracle(x, q0, s0, 700, 1200, "large, aligned q")
    for off in (1, 3):
        say("large, q offset", off)
        buf = torch.full((700 * 1200 + 8,), 0x5A, dtype=torch.uint8, device=DEV)
        q = buf[off:off + 700 * 1200].view(700, 1200)
        s = torch.empty((1, 1), dtype=torch.float32, device=DEV)
        fq.quantize(x, (700, 1200), out=(q, s))
        assert torch.equal(q, q0.view(torch.uint8)) and torch.equal(s, s0), off
        buf2 = torch.full_like(buf, 0x5A)
        q2 = buf2[off:off + 700 * 1200].view(700, 1200)
        fq.quantize_many([x, x[:350]], (700, 1200),
                         outputs=[(q2, torch.empty((1, 1), device=DEV)),
                                  (torch.empty((350, 1200), dtype=torch.uint8, device=DEV),
                                   torch.empty((1, 1), device=DEV))])
        assert torch.equal(q2, q0.view(torch.uint8)), off
        for b in (buf, buf2):
            rest = torch.cat([b[:off], b[off + 700 * 1200:]])
            assert bool((rest == 0x5A).all()), off
    # grouped call with per-tensor blocks: one scale per tensor for the C2 layer
    specs = wl.c2()
    xs = [wl.materialize(sp, DEV) for sp in specs]
    outs = fq.quantize_many(xs, (16384, 16384))
    for sp, x, (q, s) in zip(specs, xs, outs):
        assert s.shape == (1, 1)
        amax = float(x.abs().max().float())
        assert float(s[0, 0]) == float(np.float32(max(amax, np.float32(1e-10)) / 448.0)), sp.name
        q1, s1 = fq.quantize(x, (16384, 16384))
        assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), sp.name
        rows = slice(0, 64)
        q_ref, _ = oracle.quantize_with_amax(bits_np(x[rows].contiguous()), 16384, 16384,
                                             np.array([[amax]]))
        assert np.array_equal(codes_np(q[rows].contiguous()), q_ref), sp.name
        assert_properties_gpu(x, q, s, sp.M, sp.N, sp.name)


def test_grouped_large_tiles_many_tensors(gpu_lib, oracle_pool):
    """More than 128 tensors with large tiles in one grouped call (several
    grouped two-pass launches), mixed with ordinary tensors, equal single
    calls and the oracle."""
    g = torch.Generator(device=DEV).manual_seed(61)
    rng = np.random.default_rng(61)
    mats = []
    for i in range(300):
        M, N = int(rng.integers(260, 400)), int(rng.choice([264, 300, 333, 512]))
        mats.append((torch.randn((M, N), generator=g, device=DEV) * 0.05).to(torch.bfloat16))
    mats[5] = torch.zeros_like(mats[5])
    outs = fq.quantize_many(mats, (512, 512))
    for i, (x, (q, s)) in enumerate(zip(mats, outs)):
        q1, s1 = fq.quantize(x, (512, 512))
        assert torch.equal(q1.view(torch.uint8), q.view(torch.uint8)), i
        assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), i
    chk = FullOracleCheck(oracle_pool, 512, 512, "grouped large tiles")
    for i, (x, (q, s)) in enumerate(zip(mats, outs)):
        chk.add(f"[{i}]", x, q, s)
    chk.finish()


@pytest.mark.parametrize("M,N,bm,bn", [(6145, 16384, 6145, 16384),    # 3 chunks per pass-1 item, last item 1
                                      (4096, 16384, 4096, 16384),    # 2 chunks per item
                                      (8192, 8192, 4096, 2048)])     # 8 tiles of row runs, 2 per item
def test_large_tiles_chunk_grouping(gpu_lib, oracle_pool, M, N, bm, bn):
    """Large tiles where pass-1 workgroups take several chunks each (the
    host's chunks-per-workgroup above 1): single and grouped calls agree, and
    every byte and scale equals the oracle's (its two passes over pieces of
    the tiles)."""
    say("chunk grouping", M, N, bm, bn)
    g = torch.Generator(device=DEV).manual_seed(M + N)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.03).to(torch.bfloat16)
    x[M - 1, N - 1] = -2.5                                 # in the last chunk of the last tile
    q, s = fq.quantize(x, (bm, bn))
    ((qg, sg),) = fq.quantize_many([x], (bm, bn))
    assert torch.equal(q.view(torch.uint8), qg.view(torch.uint8))
    assert torch.equal(s.view(torch.int32), sg.view(torch.int32))
    chk = FullOracleCheck(oracle_pool, bm, bn, f"chunk grouping {M}x{N} [{bm},{bn}]")
    chk.add("x", x, q, s)
    chk.finish()


def test_per_tensor_vocab_matrix(gpu_lib, oracle_pool):
    """One scale for the whole 151937x4096 matrix (1.2 GB, one tile of 622M
    values, the two-pass kernels): every byte and the scale against the
    oracle (its two passes over pieces of the tile), invariants everywhere."""
    sp = [t for t in wl.c5() if t.M == 151937][0]
    x = wl.materialize(sp, DEV)
    q, s = fq.quantize(x, (sp.M, sp.N))
    amax = float(x.abs().max().float())
    assert float(s[0, 0]) == float(np.float32(max(amax, np.float32(1e-10)) / 448.0))
    assert_properties_gpu(x, q, s, sp.M, sp.N, "vocab per-tensor")
    chk = FullOracleCheck(oracle_pool, sp.M, sp.N, "vocab per-tensor")
    chk.add(sp.name, x, q, s)
    chk.finish()


@pytest.mark.parametrize("M,N", [(1024, 1024),      # 2^20 values: 128 workgroups x 4 chunks
                                 (1031, 1032),      # ragged: 65 x 8, loads past the end
                                 (2048, 4096),      # 128 x 32
                                 (4096, 4096),      # 256 x 32
                                 (1, 2 ** 21 + 8),  # one row
                                 (2 ** 17 + 3, 8)]) # eight columns
def test_per_tensor_held_in_registers(gpu_lib, M, N):
    """One scale per tensor through the kernel that holds the tensor in
    registers: equal to the oracle byte for byte (including q bytes 0..7 and
    128..135, which carry the cross-workgroup handshake during the call),
    nothing written past q, the same through the grouped call, and the same
    when every workgroup but the last computes the maximum itself."""
    say("resident", M, N)
    g = torch.Generator(device=DEV).manual_seed(M * 7 + N)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.04).to(torch.bfloat16)
    x.view(-1)[(M * N) // 2 + 5] = -1.75            # the maximum, held by one workgroup
    buf = torch.full((M * N + 256,), 0x5A, dtype=torch.uint8, device=DEV)
    q = buf[:M * N].view(M, N)
    s = torch.empty((1, 1), dtype=torch.float32, device=DEV)
    fq.quantize(x, (M, N), out=(q, s))
    assert_matches_oracle(x, q, s, M, N, f"resident {M}x{N}")
    assert bool((buf[M * N:] == 0x5A).all())
    ((qg, sg),) = fq.quantize_many([x], (M, N))
    assert torch.equal(qg.view(torch.uint8), q) and torch.equal(sg.view(torch.int32), s.view(torch.int32))
    try:
        fq.set_resident_wait_us(0)
        q0, s0 = fq.quantize(x, (M, N))
        torch.cuda.synchronize()
    finally:
        fq.set_resident_wait_us(2000)
    assert torch.equal(q0.view(torch.uint8), q) and torch.equal(s0.view(torch.int32), s.view(torch.int32))


def test_per_tensor_register_capacity(gpu_lib, oracle_pool):
    """12288x4096, the largest tensor the register-resident kernel holds on an
    MI355X (512 workgroups x 256 threads x 48 chunks), and 12289x4096, one
    row more, which takes the two-pass path: every byte and the scale against
    the oracle, invariants everywhere; a grouped call mixing both with a
    misaligned and a small tensor equals the single calls."""
    g = torch.Generator(device=DEV).manual_seed(83)
    outs = []
    xs = []
    chk = FullOracleCheck(oracle_pool, 16384, 16384, "resident capacity")
    for M in (12288, 12289):
        say("resident capacity", M)
        x = (torch.randn((M, 4096), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
        x[M - 1, 4095] = 2.25
        q, s = fq.quantize(x, (16384, 16384))
        amax = float(x.abs().max().float())
        assert amax == 2.25
        assert float(s[0, 0]) == float(np.float32(np.float32(amax) / np.float32(448.0)))
        assert_properties_gpu(x, q, s, 16384, 16384, f"capacity {M}")
        chk.add(f"{M}x4096", x, q, s)
        xs.append(x)
        outs.append((q, s))
    chk.finish()
    raw = (torch.randn(1500 * 1200 + 8, generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    mis = raw[1:1 + 1500 * 1200].view(1500, 1200)   # x not 16-byte aligned: two-pass path
    small = (torch.randn((100, 200), generator=g, device=DEV)).to(torch.bfloat16)
    group = [xs[0], mis, xs[1], small]
    got = fq.quantize_many(group, (16384, 16384))
    for i, x in enumerate(group):
        q1, s1 = outs[i // 2] if i in (0, 2) else fq.quantize(x, (16384, 16384))
        assert torch.equal(got[i][0].view(torch.uint8), q1.view(torch.uint8)), i
        assert torch.equal(got[i][1].view(torch.int32), s1.view(torch.int32)), i
    assert_matches_oracle(mis, got[1][0], got[1][1], 16384, 16384, "grouped misaligned")
    del xs, outs, got


def test_per_tensor_resident_groups(gpu_lib, oracle_pool):
    """Grouped one-scale-per-tensor calls through the persistent resident
    launch: 300 tensors of mixed sizes (three launches of up to 128 tensors,
    tensors on disjoint and wrapping workgroup ranges) equal the single calls,
    also when every workgroup but the last of each tensor computes the
    maximum itself; every byte and scale against the oracle."""
    g = torch.Generator(device=DEV).manual_seed(89)
    rng = np.random.default_rng(89)
    shapes = [(1024, 1024), (1031, 1032), (2048, 1024), (512, 4096), (4096, 1024), (1100, 3000)]
    xs = []
    for i in range(300):
        M, N = shapes[int(rng.integers(len(shapes)))]
        x = (torch.randn((M, N), generator=g, device=DEV) * float(rng.uniform(0.01, 0.1))).to(torch.bfloat16)
        x.view(-1)[int(rng.integers(M * N))] = float(rng.uniform(-3, 3))
        xs.append(x)
    xs[7] = torch.zeros_like(xs[7])
    block = (8192, 8192)
    outs = fq.quantize_many(xs, block)
    singles = [fq.quantize(x, block) for x in xs]
    for i, ((q, s), (q1, s1)) in enumerate(zip(outs, singles)):
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), i
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), i
    chk = FullOracleCheck(oracle_pool, *block, "resident groups")
    for i, (x, (q, s)) in enumerate(zip(xs, outs)):
        chk.add(f"[{i}]", x, q, s)
    chk.finish()
    try:
        fq.set_resident_wait_us(0)
        outs0 = fq.quantize_many(xs[:40], block)
        torch.cuda.synchronize()
    finally:
        fq.set_resident_wait_us(2000)
    for i, (q, s) in enumerate(outs0):
        assert torch.equal(q.view(torch.uint8), outs[i][0].view(torch.uint8)), i
        assert torch.equal(s.view(torch.int32), outs[i][1].view(torch.int32)), i


# ------------------------------------------------------------------ maximum sizes

def test_beyond_2_31_elements(gpu_lib, oracle_pool):
    """A 33000x65536 matrix (2.16e9 elements, 4.3 GB) through the [128,128],
    [1,128] and register-tile kernels and a 1 x (2^31 - 1) row through the
    general kernel, grouped [1,4096] tiles and one scale for the whole row:
    every byte and scale against the oracle (chunks of whole tile rows, or
    its two passes over pieces where a tile row is longer than a piece), and
    the dequantized tail."""
    M, N = 33000, 65536
    g = torch.Generator(device=DEV).manual_seed(59)
    x = (torch.randn((M, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    x[-1, -5:] = 3.0
    for block in [(128, 128), (1, 128), (8, 1024)]:
        bm, bn = block
        say("2^31+", block)
        q, s = fq.quantize(x, block)
        chk = FullOracleCheck(oracle_pool, bm, bn, f"2^31+ {block}")
        chk.add(f"{M}x{N}", x, q, s)
        chk.finish()
        tail = fq.dequantize(q[-bm:].contiguous(), s[-1:].contiguous(), block,
                             out_dtype=torch.bfloat16)
        want = oracle.dequantize(codes_np(q[-bm:].contiguous()), s[-1:].cpu().numpy(), bm, bn, "bf16")
        assert np.array_equal(tail.float().cpu().numpy().astype(np.float64), want)
        del q, s, tail
    del x
    torch.cuda.empty_cache()
    n = 2 ** 31 - 1
    row = (torch.randn((1, n), generator=g, device=DEV) * 0.02).to(torch.bfloat16)   # N odd: general kernel
    row[0, n - 1] = -7.0
    say("1 x 2^31-1 [1,128]")
    q, s = fq.quantize(row, (1, 128))
    assert s.shape == (1, -(-n // 128))
    assert int(q.view(torch.uint8)[0, n - 1]) == 0xFE
    chk = FullOracleCheck(oracle_pool, 1, 128, "1 x 2^31-1 [1,128]")
    chk.add("row", row, q, s)
    chk.finish()
    del q, s
    # the same row in grouped calls: [1,4096] tiles from the kernel-argument
    # table (N + bn - 1 exceeds 2^31), then one scale for the whole row
    # (grouped two-pass kernels, and the single call)
    say("1 x 2^31-1 grouped [1,4096]")
    ((q, s),) = fq.quantize_many([row], (1, 4096))
    assert s.shape == (1, -(-n // 4096))
    chk = FullOracleCheck(oracle_pool, 1, 4096, "grouped 1 x 2^31-1 [1,4096]")
    chk.add("row", row, q, s)
    chk.finish()
    del q, s
    s_ref, _ = oracle.blockwise.tile_scales_np(np.array([[7.0]]))
    for how in ("grouped", "single"):
        say("1 x 2^31-1 one scale,", how)
        if how == "grouped":
            ((q, s),) = fq.quantize_many([row], (1, n))
        else:
            q, s = fq.quantize(row, (1, n))
        assert np.array_equal(scales_bits(s), scales_bits(s_ref.astype(np.float32))), how
        chk = FullOracleCheck(oracle_pool, 1, n, f"1 x 2^31-1 one scale, {how}")
        chk.add("row", row, q, s)
        chk.finish()
        del q, s
