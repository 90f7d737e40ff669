"""Oracle: exact decoding of the block-quantised expert formats (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats (each a structure of arrays: a code array and a scale array, blocks run
along a matrix row's reduction dimension, per the GGUF convention that the model
card's "Sources" section fixes by saying the tensors are copied unchanged from
GGUF files):

* Q8_0: 32-element blocks, int8 codes, one IEEE binary16 scale per block
  (34 bytes per 32 weights).  Named as a covered down format in "What was
  changed" of the UD-IQ2_XS (L4 fix) page.
* IQ4_NL: 32-element blocks, 4-bit indices into the 16-entry non-linear int8
  codebook, one binary16 scale (18 bytes per 32 weights = 4.5 bits per weight,
  the figure "What was changed" gives).  Within a block's 16 code bytes, the low
  nibble of byte j is element j and the high nibble is element j + 16.
* NVFP4-style: 16-element blocks of FP4 E2M1 codes (element 2i in the low nibble
  of byte i), one FP8 E4M3 block scale, one fp32 scale per (expert, matrix).  The
  pages' benchmark ("Benchmark: seven engines on one RTX 5090", "Engine
  provenance") runs NVIDIA's NVFP4 routed experts bit-exact.
* Q5_1: 32-element blocks of 5-bit unsigned codes with a binary16 step d and a
  binary16 offset m, w = d * q + m, from ggml's public Q5_1 definition (a
  covered down format in "What was changed").  The low 4 bits of the codes use
  the IQ4_NL nibble order (16 bytes); the fifth bit of element e is bit e of a
  32-bit word.  Structure of arrays: the 16 code bytes per block, and one
  8-byte record per block holding d, m and that word (little-endian), 24 bytes
  per 32 weights = 6 bits per weight.

Every value is computed from its closed form with exact float64 arithmetic.
"""

import numpy as np

# The IQ4_NL codebook (GGUF's non-linear 4-bit table), as the workload
# definition prints it.
IQ4_NL_CODEBOOK = np.array(
    [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113],
    dtype=np.float64)

Q8_0_BLOCK = 32
IQ4_NL_BLOCK = 32
NVFP4_BLOCK = 16


def fp16_bits_to_float(bits):
    """IEEE 754 binary16 -> float64, from the closed form.

    sign s, 5-bit exponent e (bias 15), 10-bit fraction m:
    e == 0: (-1)^s * m * 2^-24;  0 < e < 31: (-1)^s * (1024 + m) * 2^(e - 25);
    e == 31: inf (m == 0) or NaN.  Pinned exhaustively against numpy.float16.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -24),
                   np.ldexp((1024 + m).astype(np.float64), (e - 25).astype(np.int64)))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def e4m3_bits_to_float(bits):
    """OCP FP8 E4M3 -> float64, from the closed form.

    sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  e == 0 is
    subnormal m * 2^-9; otherwise (8 + m) * 2^(e - 10); S.1111.111 is NaN and
    there is no infinity (largest finite value 448).  Pinned exhaustively
    against torch.float8_e4m3fn.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFF
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e2m1_bits_to_float(nibbles):
    """OCP MX FP4 E2M1 -> float64, from the closed form.

    sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.  e == 0 is
    subnormal m * 0.5; otherwise (2 + m) * 2^(e - 2).  Magnitudes are
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Pinned against torch.float4_e2m1fn_x2.
    """
    n = np.asarray(nibbles).astype(np.int64) & 0xF
    s = (n >> 3) & 1
    e = (n >> 1) & 0x3
    m = n & 1
    mag = np.where(e == 0, 0.5 * m,
                   np.ldexp((2 + m).astype(np.float64), (e - 2).astype(np.int64)))
    return np.where(s == 1, -mag, mag)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits; NaN is kept quiet.  Pinned against torch's
    float32 -> bfloat16 conversion on all patterns of a large random sample and
    on every tie case.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(f)
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_bits_to_float(bits):
    """bfloat16 bit pattern -> float64 (exact: the pattern is the top half of a float32)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """float64 -> nearest bfloat16 value (round to nearest, ties to even),
    rounded once from the float64 value, returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range: normal
    values in [2^-126, 2^128) have a spacing of 2^(e - 7) in the binade
    [2^e, 2^(e+1)); below 2^-126 the spacing is 2^-133 (subnormals).  x is
    divided by its spacing (a power of two, exact), rounded to an integer
    with ties to even, and scaled back; a result at or beyond 2^128 is an
    overflow to infinity.  Pinned against an exact rational rounding,
    including inputs that a float32 intermediate would round twice.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)                     # |x| = m * 2^e2, m in [0.5, 1)
    ex = np.maximum(e2 - 1, -126)            # binade exponent, clamped at the subnormal range
    sp = np.ldexp(1.0, (ex - 7).astype(np.int64))
    r = np.rint(xf / sp) * sp                # rint rounds ties to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def dequant_q8_0(codes, scales):
    """Q8_0 block dequantisation: w = code * fp16(scale), exact in float64.

    codes: int8 [..., rows, cols]; scales: uint16 binary16 bits [..., rows, cols/32].
    The product of an int8 and a binary16 has at most 19 significant bits, so it
    is also exact in float32.
    """
    c = np.asarray(codes).astype(np.int8).astype(np.float64)
    d = fp16_bits_to_float(scales)
    rows_shape = c.shape[:-1]
    nb = c.shape[-1] // Q8_0_BLOCK
    c = c.reshape(rows_shape + (nb, Q8_0_BLOCK))
    return (c * d[..., None]).reshape(rows_shape + (nb * Q8_0_BLOCK,))


def iq4_nl_unpack(codes):
    """IQ4_NL code bytes [..., rows, cols/2] -> nibble indices [..., rows, cols].

    Per 16-byte block: element j is the low nibble of byte j, element j + 16 the
    high nibble of byte j (the GGUF layout).
    """
    b = np.asarray(codes).astype(np.uint8)
    rows_shape = b.shape[:-1]
    nb = b.shape[-1] // 16
    b = b.reshape(rows_shape + (nb, 16))
    lo = b & 0x0F
    hi = b >> 4
    idx = np.concatenate([lo, hi], axis=-1)  # elements 0..15 then 16..31
    return idx.reshape(rows_shape + (nb * 32,))


def dequant_iq4_nl(codes, scales):
    """IQ4_NL block dequantisation: w = codebook[nibble] * fp16(scale), exact.

    codes: uint8 [..., rows, cols/2]; scales: uint16 binary16 bits [..., rows, cols/32].
    """
    idx = iq4_nl_unpack(codes)
    v = IQ4_NL_CODEBOOK[idx]
    d = fp16_bits_to_float(scales)
    rows_shape = v.shape[:-1]
    nb = v.shape[-1] // IQ4_NL_BLOCK
    v = v.reshape(rows_shape + (nb, IQ4_NL_BLOCK))
    return (v * d[..., None]).reshape(rows_shape + (nb * IQ4_NL_BLOCK,))


def nvfp4_unpack(codes):
    """NVFP4 code bytes [..., rows, cols/2] -> E2M1 nibbles [..., rows, cols]
    (element 2i in the low nibble of byte i, element 2i + 1 in the high nibble)."""
    b = np.asarray(codes).astype(np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def dequant_nvfp4(codes, scales, tensor_scale):
    """NVFP4-style dequantisation: w = fp32_RNE(e2m1(code) * e4m3(block scale) * ts).

    codes: uint8 [rows, cols/2]; scales: uint8 E4M3 bits [rows, cols/16];
    tensor_scale: one float32 for this (expert, matrix).  e2m1 * e4m3 has at most
    6 significant bits and is exact; multiplying by the float32 tensor scale is
    exact in float64 (at most 30 bits) and is then rounded once to float32.
    """
    v = e2m1_bits_to_float(nvfp4_unpack(codes))
    s = e4m3_bits_to_float(scales)
    rows_shape = v.shape[:-1]
    nb = v.shape[-1] // NVFP4_BLOCK
    v = v.reshape(rows_shape + (nb, NVFP4_BLOCK))
    a = (v * s[..., None]).reshape(rows_shape + (nb * NVFP4_BLOCK,))
    ts = np.float64(np.float32(tensor_scale))
    return (a * ts).astype(np.float32).astype(np.float64)


Q5_1_BLOCK = 32


def q5_1_unpack(codes, records):
    """Q5_1 code bytes [..., rows, cols/2] and 8-byte block records
    [..., rows, cols/32 * 8] -> (q [..., rows, cols] in 0..31, d and m
    [..., rows, cols/32] as float64).

    Record bytes 0-1: binary16 d; 2-3: binary16 m; 4-7: the high-bit word,
    little-endian; bit e of that word is the fifth bit of block element e.
    """
    low = iq4_nl_unpack(codes).astype(np.int64)  # the same 4-bit packing
    rec = np.asarray(records).astype(np.int64)
    rows_shape = rec.shape[:-1]
    nb = rec.shape[-1] // 8
    rec = rec.reshape(rows_shape + (nb, 8))
    d = fp16_bits_to_float(rec[..., 0] | (rec[..., 1] << 8))
    m = fp16_bits_to_float(rec[..., 2] | (rec[..., 3] << 8))
    word = rec[..., 4] | (rec[..., 5] << 8) | (rec[..., 6] << 16) | (rec[..., 7] << 24)
    high = (word[..., None] >> np.arange(Q5_1_BLOCK)) & 1       # [..., nb, 32]
    q = low.reshape(rows_shape + (nb, Q5_1_BLOCK)) + 16 * high
    return q.reshape(rows_shape + (nb * Q5_1_BLOCK,)), d, m


def dequant_q5_1(codes, records):
    """Q5_1 block dequantisation: w = d * q + m, exact in float64 (d * q has at
    most 16 significant bits, and the sum of two values of the binary16 range
    needs at most 45)."""
    q, d, m = q5_1_unpack(codes, records)
    rows_shape = q.shape[:-1]
    nb = q.shape[-1] // Q5_1_BLOCK
    q = q.reshape(rows_shape + (nb, Q5_1_BLOCK)).astype(np.float64)
    return (q * d[..., None] + m[..., None]).reshape(rows_shape + (nb * Q5_1_BLOCK,))


def dequant(qtype, codes, scales, tensor_scale=None):
    """Dispatch on the format name ('q8_0', 'iq4_nl', 'nvfp4', 'q5_1') for one expert matrix."""
    if qtype == "q8_0":
        return dequant_q8_0(codes, scales)
    if qtype == "iq4_nl":
        return dequant_iq4_nl(codes, scales)
    if qtype == "nvfp4":
        return dequant_nvfp4(codes, scales, tensor_scale)
    if qtype == "q5_1":
        return dequant_q5_1(codes, scales)
    raise ValueError(f"unknown format {qtype!r}")


def bytes_per_matrix(qtype, rows, cols):
    """Algorithmic bytes of one expert matrix in the given format (codes + scales
    [+ 4-byte tensor scale]).  IQ4_NL: 18 B per 32 weights (4.5 bits per weight)."""
    n = rows * cols
    if qtype == "q8_0":
        return n // 32 * 34
    if qtype == "iq4_nl":
        return n // 32 * 18
    if qtype == "nvfp4":
        return n // 16 * 9 + 4
    if qtype == "q5_1":
        return n // 32 * 24
    raise ValueError(qtype)
