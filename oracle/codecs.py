"""Reference storage codecs and the fp8 per-block scale rule (test
infrastructure only).

The pages name 16-bit storage ("2 bytes per number", [KPF] "Opening the
hood"; [DF] cache-size formula) and 8-bit floating-point storage for the
cache ([KVFA] memory-cost section; [DF] number-format paragraph), but fix
neither the 8-bit format nor its scaling.  The readings used here:

* 16-bit: bf16 and fp16, round-to-nearest-even from float32.
* 8-bit: the OCP "E4M3FN" format (1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, no infinities, the all-ones pattern is NaN, largest finite
  value 448), encoded with round-to-nearest-even and saturation to +-448.
* One float32 scale per (layer, block, kv head), separately for K and V:
  s = absmax / 448 over the rows written so far to that 16-row slab; a code
  stores round(x / s).  The arithmetic of the rule is float32 (IEEE single
  division and multiplication, correctly rounded), and numpy's float32 scalar
  and array operations are exactly that.
"""
import math

import numpy as np

E4M3_MAX = 448.0
F32 = np.float32


# --------------------------------------------------------------------- bf16
def bf16_bits_from_f32(x):
    """Round float32 values to bf16, returning the 16-bit patterns (uint16).

    Round to nearest, ties to even, done on the bit pattern: add 0x7FFF plus
    the lowest kept bit, then drop the low 16 bits.  NaN maps to a quiet NaN.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b):
    """Widen bf16 bit patterns (uint16) to float64, exactly."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b):
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


# --------------------------------------------------------------------- fp16
def f16_bits_from_f32(x):
    """Round float32 to IEEE binary16 (numpy's cast is round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- fp8 e4m3fn
def e4m3_value(code):
    """Exact real value of one 8-bit E4M3FN pattern (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6          # subnormal: 0.m x 2^-6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)   # normal: 1.m x 2^(e-7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(x):
    """Encode finite values (given exactly, e.g. float32) to E4M3FN codes.

    Round to nearest, ties to even, with magnitudes at or above 448 saturated
    to 448 (the pattern 0x7E); the sign bit is copied, so a negative value
    that rounds to zero gives 0x80.  Works in float64, where every step is
    exact for float32 inputs: below 2^-6 the representable magnitudes are
    spaced 2^-9 apart (subnormals); between 2^e and 2^(e+1) they are spaced
    2^(e-3).  Codes of consecutive magnitudes are consecutive integers, so a
    mantissa that rounds up to the next power of two carries into the
    exponent field by plain addition.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no encoding in this codec")
    sign = np.where(np.signbit(x), 0x80, 0x00)
    a = np.abs(x)
    _, E = np.frexp(a)                     # a = f * 2^E with f in [0.5, 1)
    e = np.where(a < 2.0 ** -6, -6, E - 1)  # exponent of the spacing band
    n = np.rint(a / np.exp2(e - 3))        # ties to even
    code = np.where(a < 2.0 ** -6,
                    n,                     # subnormal band: code = n (0..8)
                    ((e + 7) << 3) + n - 8)
    code = np.where(a >= E4M3_MAX, 0x7E, np.minimum(code, 0x7E))
    return (sign | code.astype(np.int64)).astype(np.uint8)


def e4m3_decode(codes):
    """Exact decode of E4M3FN codes to float64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp8_slab_write(codes, scale, r0, new_rows):
    """Write rows r0 .. r0+n-1 of one (block, kv head) slab of an fp8 cache.

    codes: uint8 [16, d] current codes of the slab (rows < r0 are live);
    scale: float32 current scale of the slab (ignored when r0 == 0);
    new_rows: [n, d] float32 values to store (bf16 inputs widened exactly).
    Returns (codes, scale) after the write.

    The scale stays absmax/448 over every row written so far.  Because
    float32 division by 448 is monotonic, max(s_old, absmax(new)/448) is
    exactly absmax(all rows)/448, so the rule never needs the old absmax.
    When the scale grows, the live rows are re-encoded from their decoded
    values: x = fl32(decode(code) * s_old), code' = encode(fl32(x / s_new)).
    A slab whose rows are all zero has scale 0 and every code stays +-0.
    """
    codes = np.array(codes, dtype=np.uint8, copy=True)
    new_rows = np.asarray(new_rows, dtype=np.float32)
    amax = F32(np.max(np.abs(new_rows))) if new_rows.size else F32(0.0)
    s_new = F32(amax / F32(E4M3_MAX))
    if r0 == 0:
        s = s_new
    else:
        s_old = F32(scale)
        s = F32(max(s_old, s_new))
        if s > s_old:
            for r in range(r0):
                x = (e4m3_decode(codes[r]).astype(np.float32) * s_old).astype(np.float32)
                codes[r] = e4m3_encode((x / s).astype(np.float32))
    for i in range(new_rows.shape[0]):
        row = new_rows[i]
        q = (row / s).astype(np.float32) if s > 0 else row
        codes[r0 + i] = e4m3_encode(q)
    return codes, s


# ------------------------------------------------------------------ int4
# The pages name an int4 cache only in passing ([KVFA] memory-cost section:
# servers quantize the cache to fp8 or int4 first).  Reading: symmetric
# integers -7 .. 7 (the code -8 is never produced) times one float32 scale
# per (layer, block, kv head) slab, the same slab granularity and growth rule
# as the fp8 cache with 7 in place of 448.  Two codes per byte, element 2i in
# the low nibble, two's complement.
INT4_MAX = 7


def int4_encode(y):
    """Codes of already-scaled float32 values: round to nearest, ties to
    even, clamped to -7 .. 7.  Returns int8 codes."""
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("NaN has no encoding in this codec")
    return np.clip(np.rint(y), -INT4_MAX, INT4_MAX).astype(np.int8)


def int4_decode(codes):
    """Exact value of int4 codes (before the scale)."""
    return np.asarray(codes, dtype=np.float64)


def int4_slab_write(codes, scale, r0, new_rows):
    """Write rows r0 .. r0+n-1 of one (block, kv head) slab of an int4 cache.

    codes: int8 [16, d] current codes of the slab (rows < r0 are live);
    scale: float32 current scale (ignored when r0 == 0); new_rows: [n, d]
    float32 values.  Returns (codes, scale).  The scale is absmax/7 over every
    row written so far, kept as max(s_old, absmax(new)/7); when it grows the
    live rows are re-encoded: x = fl32(code * s_old), code' =
    encode(fl32(x / s_new)).  An all-zero slab has scale 0 and codes 0.
    """
    codes = np.array(codes, dtype=np.int8, copy=True)
    new_rows = np.asarray(new_rows, dtype=np.float32)
    amax = F32(np.max(np.abs(new_rows))) if new_rows.size else F32(0.0)
    s_new = F32(amax / F32(INT4_MAX))
    if r0 == 0:
        s = s_new
    else:
        s_old = F32(scale)
        s = F32(max(s_old, s_new))
        if s > s_old:
            for r in range(r0):
                x = (codes[r].astype(np.float32) * s_old).astype(np.float32)
                codes[r] = int4_encode((x / s).astype(np.float32))
    for i in range(new_rows.shape[0]):
        row = new_rows[i]
        q = (row / s).astype(np.float32) if s > 0 else row
        codes[r0 + i] = int4_encode(q)
    return codes, s


def int4_pack(codes, axis=-1):
    """Pack int8 codes two per byte along `axis` (even index in the low
    nibble).  The axis length must be even."""
    c = np.moveaxis(np.asarray(codes, dtype=np.int8), axis, -1).astype(np.uint8) & 0x0F
    packed = c[..., 0::2] | (c[..., 1::2] << 4)
    return np.moveaxis(packed.astype(np.uint8), -1, axis)


def int4_unpack(packed, axis=-1):
    """Inverse of int4_pack: int8 codes."""
    p = np.moveaxis(np.asarray(packed, dtype=np.uint8), axis, -1)
    lo = (p & 0x0F).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo).astype(np.int8)
    hi = np.where(hi > 7, hi - 16, hi).astype(np.int8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.moveaxis(out, -1, axis)
