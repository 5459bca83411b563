"""OCP 8-bit float e4m3fn, decoded and encoded from the format's definition.

The pages only say that KV may be stored in 8 bits or fewer ("07｜…内部过程",
Q026 follow-up on KV quantisation; "03. KV Cache…", table of remedies, row
"每个数存得更小"). The format, the scale granularity and the rounding are this
library's reading:

* e4m3fn: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
  field 0 is subnormal (m/8 · 2^-6); S.1111.111 is NaN; there is no infinity;
  the largest finite magnitude is 1.75 · 2^8 = 448.
* encode: round to nearest, ties to even, and saturate: any magnitude that
  rounds above 448 (infinity included) becomes 448. NaN encodes as 0x7f with
  the input's sign bit.
* quantised value: e4m3(fp32(x · inv_scale)); dequantised value: e4m3 · scale,
  one fp32 scale per KV head for K and one for V.
"""

import math

import numpy as np


def decode(code):
    """Exact value of one e4m3fn byte (float; NaN for the NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table():
    """All 256 codes as float64."""
    return np.array([decode(c) for c in range(256)], dtype=np.float64)


def _rne(x):
    """Round a non-negative float64 to the nearest integer, ties to even."""
    f = math.floor(x)
    r = x - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


def encode_one(x):
    """Round-to-nearest-even, saturating encode of one real value."""
    x = float(x)
    if math.isnan(x):
        return 0xFF if math.copysign(1.0, x) < 0 else 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a == 0.0:
        return sign
    if math.isinf(a):
        return sign | 0x7E
    # exponent of the leading bit; below 2^-6 the spacing is fixed at 2^-9
    e = math.frexp(a)[1] - 1                      # a in [2^e, 2^(e+1))
    e = max(e, -6)
    step = 2.0 ** (e - 3)                          # spacing of 3-bit mantissas
    q = _rne(a / step)                             # exact: a/step is a power-of-two scaling
    if e == -6 and q < 8:                          # subnormal (or zero)
        code = q
    else:
        if q == 16:                                # rounded up into the next binade
            e += 1
            q = 8
        code = ((e + 7) << 3) | (q - 8)
    if code > 0x7E:                                # above 448 (or the NaN slot): saturate
        code = 0x7E
    return sign | code


def encode(x):
    """Vectorised wrapper over encode_one; returns uint8 with x's shape."""
    x = np.asarray(x)
    flat = [encode_one(v) for v in x.reshape(-1).tolist()]
    return np.array(flat, dtype=np.uint8).reshape(x.shape)


def quantize(x, inv_scale):
    """Stored byte for a cache value: e4m3(fp32(fp32(x) · fp32(inv_scale)))."""
    prod = np.asarray(x, dtype=np.float32) * np.float32(inv_scale)
    return encode(prod.astype(np.float32))


def dequantize(codes, scale):
    """Value the attention sees for stored bytes: decode(code) · scale, in float64."""
    table = decode_table()
    return table[np.asarray(codes, dtype=np.int64)] * np.float64(np.float32(scale))


def _bf16_values():
    """float32 value of every 16-bit bf16 pattern (pattern << 16 reinterpreted)."""
    bits = (np.arange(65536, dtype=np.uint32) << 16).astype(np.uint32)
    return bits.view(np.float32)


_TABLES = {}


def quantize_bf16_bits(bits, inv_scale):
    """quantize() for bf16 inputs given as raw uint16 patterns. Same definition,
    evaluated once for each of the 65536 patterns and then looked up, so large
    caches quantise in reasonable time."""
    key = float(np.float32(inv_scale))
    table = _TABLES.get(key)
    if table is None:
        with np.errstate(over="ignore", invalid="ignore"):
            table = quantize(_bf16_values(), np.float32(inv_scale))
        _TABLES[key] = table
    return table[np.asarray(bits, dtype=np.uint16).astype(np.int64)]
