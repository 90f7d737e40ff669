"""Pins for the oracle's format decoders (CPU only).

Each decoder is checked against something other than itself: numpy / torch
dtype conversions, exhaustive tables, exact rational arithmetic and the golden
fixtures under tests/golden/ (each cites its source)."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- scalar types

def test_fp16_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = F.fp16_bits_to_float(bits)
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(got[~nan_ref]))


def test_e4m3_exhaustive_against_torch():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3_bits_to_float(np.arange(256))
    nan_ref = np.isnan(ref)
    assert nan_ref.sum() == 2  # S.1111.111 only
    assert np.array_equal(nan_ref, np.isnan(got))
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    assert np.nanmax(got) == 448.0


def test_e2m1_against_golden_table():
    table = _read_golden("e2m1_values.txt")
    assert len(table) == 16
    for code, val in table:
        c = int(code, 16)
        got = F.e2m1_bits_to_float(np.array([c]))[0]
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), (c, got, want)


def test_e2m1_widened_into_e4m3_agrees_with_torch():
    # A normal E2M1 value (s, e, m) equals the E4M3 value (s, e + 6, m << 2):
    # both biases differ by 6.  Independent of the golden table above.
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e == 0:
            continue
        b = (s << 7) | ((e + 6) << 3) | (m << 2)
        ref = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert F.e2m1_bits_to_float(np.array([c]))[0] == ref


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add every tie pattern around a few exponents
    ties = np.array([(e << 23) | (m << 16) | 0x8000 for e in (1, 100, 127, 200, 254) for m in range(0, 128, 7)],
                    dtype=np.uint32)
    bits = np.concatenate([bits, ties, ties | 0x80000000])
    f = bits.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f32_to_bf16_bits(f)
    assert np.array_equal(ref, got)


def test_bf16_round_once_against_exact_rationals():
    """round_to_bf16 rounds the float64 value once (ties to even), checked
    against exact rational rounding on random values over the whole range,
    every exact midpoint kind, subnormals, overflow, and values just off a
    midpoint that a float32 intermediate would first round onto it."""
    import math
    from fractions import Fraction

    import exact_round as ER

    rng = np.random.default_rng(8)
    vals = list(rng.normal(size=400) * np.exp2(rng.uniform(-140, 130, size=400)))
    vals += [0.0, -0.0, 1.0, -3.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126, 2.0 ** -127 * 1.5]
    # largest finite bf16, just below and at the overflow midpoint
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    vals += [mx, mx + 2.0 ** 119 - 2.0 ** 90, mx + 2.0 ** 119, -(mx + 2.0 ** 119)]
    for e in (-130, -126, -60, -1, 0, 7, 100, 127):
        for m in range(128, 256, 9):
            b = m * 2.0 ** (e - 7)             # a bf16 value with significand m
            mid = b + 2.0 ** (e - 8)           # the midpoint above it
            vals += [mid, -mid, mid + mid * 2.0 ** -40, mid - mid * 2.0 ** -40]
    x = np.array(vals, dtype=np.float64)
    got = F.round_to_bf16(x)
    for v, g in zip(x, got):
        want = ER.rne(Fraction(float(v)), ER.BF16)
        if isinstance(want, float) and math.isinf(want):
            assert math.isinf(g) and (g > 0) == (want > 0), v
        else:
            assert math.isfinite(g) and Fraction(float(g)) == want, (v, g, float(want))
    assert np.isnan(F.round_to_bf16(np.array([np.nan]))[0])
    assert np.array_equal(F.round_to_bf16(np.array([np.inf, -np.inf])), np.array([np.inf, -np.inf]))


def test_numpy_float16_conversion_rounds_once():
    """numpy's float64 -> float16 conversion (the GPU tests' reference for the
    prefill fp16 weight tile) is one round-to-nearest-even, overflow to inf,
    checked against exact rational rounding."""
    import math
    from fractions import Fraction

    import exact_round as ER

    rng = np.random.default_rng(12)
    vals = list(rng.normal(size=300) * np.exp2(rng.uniform(-28, 17, size=300)))
    for m in range(1024, 2048, 37):
        for e in (-24, -15, -14, 0, 15):
            b = m * 2.0 ** (e - 10)
            mid = b + 2.0 ** (e - 11)
            vals += [mid, mid + mid * 2.0 ** -30, mid - mid * 2.0 ** -30]
    vals += [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 3 * 2.0 ** -26]
    for v in vals:
        g = float(np.float16(v))
        want = ER.rne(Fraction(v), ER.F16)
        if isinstance(want, float):
            assert math.isinf(g) and (g > 0) == (want > 0), v
        else:
            assert math.isfinite(g) and Fraction(g) == want, (v, g, float(want))


# ---------------------------------------------------------------- block formats

def test_block_sizes_match_golden():
    for fmt, n_el, n_bytes, bpw in _read_golden("format_sizes.txt"):
        n_el, n_bytes, bpw = int(n_el), int(n_bytes), float(bpw)
        rows, cols = 4, 128
        total = F.bytes_per_matrix(fmt, rows, cols)
        extra = 4 if fmt == "nvfp4" else 0  # one fp32 tensor scale per matrix
        assert total - extra == rows * cols // n_el * n_bytes
        assert (total - extra) * 8 / (rows * cols) == bpw


def test_iq4_nl_codebook_matches_golden():
    table = _read_golden("iq4_nl_codebook.txt")
    want = np.array([int(v) for _, v in table], dtype=np.float64)
    assert np.array_equal(F.IQ4_NL_CODEBOOK, want)
    assert np.all(np.diff(want) > 0)


def _fp16_exact(bits):
    """binary16 value as an exact Fraction (independent bit decode)."""
    b = int(bits)
    s = -1 if b >> 15 else 1
    e = (b >> 10) & 31
    m = b & 1023
    if e == 0:
        return s * Fraction(m, 2 ** 24)
    return s * Fraction(1024 + m) * Fraction(2) ** (e - 25)


def test_q8_0_all_codes_times_sampled_scales_exact():
    rng = np.random.default_rng(1)
    finite = [b for b in range(65536) if ((b >> 10) & 31) != 31]
    scales = rng.choice(finite, size=64, replace=False).astype(np.uint16)
    scales = np.concatenate([scales, np.array([0x0000, 0x8000, 0x0001, 0x7BFF, 0x3C00], dtype=np.uint16)])
    codes = np.tile(np.arange(-128, 128, dtype=np.int16), 1).astype(np.int8)  # 256 codes = 8 blocks
    for s in scales:
        c = codes.reshape(1, 256)
        sc = np.full((1, 8), s, dtype=np.uint16)
        got = F.dequant_q8_0(c, sc)[0]
        exact = _fp16_exact(s)
        for i in range(256):
            assert Fraction(got[i]) == int(codes[i]) * exact


def test_iq4_nl_nibble_order_and_exact_values():
    # byte j of a block: low nibble = element j, high nibble = element j + 16
    rng = np.random.default_rng(2)
    idx = rng.integers(0, 16, size=(3, 64))  # 3 rows, 2 blocks
    codes = np.zeros((3, 32), dtype=np.uint8)
    for r in range(3):
        for b in range(2):
            for j in range(16):
                codes[r, 16 * b + j] = idx[r, 32 * b + j] | (idx[r, 32 * b + j + 16] << 4)
    scale_bits = np.array([[0x3C00, 0xB800], [0x1234, 0x0003], [0x0000, 0x7000]], dtype=np.uint16)
    got = F.dequant_iq4_nl(codes, scale_bits)
    table = [int(v) for _, v in _read_golden("iq4_nl_codebook.txt")]
    for r in range(3):
        for i in range(64):
            want = table[idx[r, i]] * _fp16_exact(scale_bits[r, i // 32])
            assert Fraction(got[r, i]) == want


def test_iq4_nl_every_code_every_scale_class():
    # all 256 code bytes under one scale: each byte decodes its two nibbles
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)  # 16 rows, one block each
    s = np.full((16, 1), 0x2E66, dtype=np.uint16)
    got = F.dequant_iq4_nl(codes, s)
    cb = [int(v) for _, v in _read_golden("iq4_nl_codebook.txt")]
    d = _fp16_exact(0x2E66)
    for r in range(16):
        for j in range(16):
            byte = 16 * r + j
            assert Fraction(got[r, j]) == cb[byte & 15] * d
            assert Fraction(got[r, j + 16]) == cb[byte >> 4] * d


def _f32_round(fr):
    """Round an exact Fraction to the nearest float32 (ties to even), independently
    of numpy: scale into [2^23, 2^24) and round the integer mantissa."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = a / Fraction(2) ** (e - 23)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** (e - 23))


def test_nvfp4_exact_products_then_one_fp32_rounding():
    rng = np.random.default_rng(3)
    cols = 64
    codes = rng.integers(0, 256, size=(4, cols // 2), dtype=np.uint8)
    sc = rng.integers(0, 0x7F, size=(4, cols // 16), dtype=np.uint8)  # finite, non-negative E4M3
    sc[0, 0] = 0x7E  # 448
    sc[1, 1] = 0x01  # smallest subnormal
    ts = np.float32(rng.uniform(1e-5, 1e-3))
    got = F.dequant_nvfp4(codes, sc, ts)
    e2 = [float(v) for _, v in _read_golden("e2m1_values.txt")]
    for r in range(4):
        for i in range(cols):
            byte = codes[r, i // 2]
            nib = (byte & 15) if i % 2 == 0 else (byte >> 4)
            sb = torch.tensor([sc[r, i // 16]], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
            exact = Fraction(e2[nib]) * Fraction(sb) * Fraction(float(ts))
            assert got[r, i] == _f32_round(exact), (r, i)


def test_zero_scale_blocks_decode_to_zero():
    codes8 = np.random.default_rng(4).integers(-127, 128, size=(2, 64)).astype(np.int8)
    z = np.zeros((2, 2), dtype=np.uint16)
    assert np.all(F.dequant_q8_0(codes8, z) == 0)
    codes4 = np.random.default_rng(5).integers(0, 256, size=(2, 32)).astype(np.uint8)
    assert np.all(F.dequant_iq4_nl(codes4, z) == 0)
    assert np.all(F.dequant_nvfp4(codes4, np.zeros((2, 4), np.uint8), np.float32(0.5)) == 0)


# ---------------------------------------------------------------- Q5_1

def _q5_1_record(d_bits, m_bits, word):
    return np.array([d_bits & 0xFF, d_bits >> 8, m_bits & 0xFF, m_bits >> 8,
                     word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF, word >> 24], dtype=np.uint8)


def _q5_1_block(q):
    """Pack 32 five-bit codes into (16 code bytes, high-bit word) by the layout:
    low nibble of byte j = element j, high nibble = element j + 16, bit e of the
    word = the fifth bit of element e."""
    q = np.asarray(q, dtype=np.int64)
    codes = ((q[:16] & 15) | ((q[16:] & 15) << 4)).astype(np.uint8)
    word = int(sum(int((q[e] >> 4) & 1) << e for e in range(32)))
    return codes, word


def test_q5_1_every_code_at_every_position_exact():
    """Every code 0..31 at every block position, with d and m over signs,
    subnormals, zero and the largest binary16 values, against exact rationals."""
    scales = [0x3C00, 0xBC00, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x0000, 0x2E66, 0xB123]
    rng = np.random.default_rng(13)
    codes, recs, want = [], [], []
    for shift in range(32):
        q = (np.arange(32) + shift) % 32
        c, word = _q5_1_block(q)
        d_bits = scales[shift % len(scales)]
        m_bits = scales[(3 * shift + 1) % len(scales)] if shift % 4 else int(rng.integers(0, 0x7C00))
        codes.append(c)
        recs.append(_q5_1_record(d_bits, m_bits, word))
        d = Fraction(float(np.uint16(d_bits).view(np.float16)))
        m = Fraction(float(np.uint16(m_bits).view(np.float16)))
        want.append([d * int(v) + m for v in q])
    codes = np.stack(codes)[None]            # [1 row, 32 blocks * 16]
    codes = codes.reshape(1, -1)
    recs = np.stack(recs).reshape(1, -1)
    got = F.dequant_q5_1(codes, recs)
    flat = [x for blk in want for x in blk]
    assert len(flat) == got.shape[1]
    for g, w in zip(got[0], flat):
        assert Fraction(float(g)) == w


def test_q5_1_high_bit_and_nibble_order():
    """One set bit of the high-bit word raises exactly its element by 16 d; a
    nibble in byte j lands at element j (low) or j + 16 (high)."""
    d_bits, m_bits = 0x3800, 0x3400  # 0.5, 0.25
    base_codes = np.zeros((1, 16), np.uint8)
    base = F.dequant_q5_1(base_codes, _q5_1_record(d_bits, m_bits, 0)[None])[0]
    assert np.all(base == 0.25)
    for e in (0, 1, 7, 15, 16, 17, 30, 31):
        w = F.dequant_q5_1(base_codes, _q5_1_record(d_bits, m_bits, 1 << e)[None])[0]
        diff = w - base
        assert diff[e] == 8.0 and np.count_nonzero(diff) == 1
    for j in (0, 5, 15):
        c = np.zeros((1, 16), np.uint8)
        c[0, j] = 0x93  # low nibble 3, high nibble 9
        w = F.dequant_q5_1(c, _q5_1_record(d_bits, m_bits, 0)[None])[0]
        assert w[j] == 0.5 * 3 + 0.25 and w[j + 16] == 0.5 * 9 + 0.25
        assert np.count_nonzero(w - base) == 2


def test_q5_1_zero_step_and_offset_decode_to_zero():
    rng = np.random.default_rng(14)
    c = rng.integers(0, 256, size=(3, 64)).astype(np.uint8)
    recs = np.concatenate([_q5_1_record(0, 0x8000, int(rng.integers(0, 2 ** 32)))
                           for _ in range(12)]).reshape(3, 32)
    assert np.all(F.dequant_q5_1(c, recs) == 0)


def test_q5_1_planted_mistakes_are_caught(monkeypatch):
    # the high bit of element j + 16 taken from bit j
    def bad_unpack(codes, records):
        q, d, m = orig(codes, records)
        rows_shape = q.shape[:-1]
        nb = q.shape[-1] // 32
        q = q.reshape(rows_shape + (nb, 32)).copy()
        q[..., 16:] = (q[..., 16:] & 15) | (q[..., :16] & 16)
        return q.reshape(rows_shape + (nb * 32,)), d, m
    orig = F.q5_1_unpack
    monkeypatch.setattr(F, "q5_1_unpack", bad_unpack)
    with pytest.raises(AssertionError):
        test_q5_1_high_bit_and_nibble_order()
    monkeypatch.undo()
    # step and offset swapped
    def bad_unpack2(codes, records):
        q, d, m = orig(codes, records)
        return q, m, d
    monkeypatch.setattr(F, "q5_1_unpack", bad_unpack2)
    with pytest.raises(AssertionError):
        test_q5_1_every_code_at_every_position_exact()
    monkeypatch.undo()
