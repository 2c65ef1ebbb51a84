"""Per-32-element block quantization to MXFP4 / MXFP8 with E8M0 scales.

Oracle (test infrastructure).  Follows, in order, the steps of the per-group
dynamic quantization on the Day-0 page (Day 0 LLM Inference Support, section
V "Engineering Implementation Details", the per-group quantization listing,
and section III.3.2 "MXFP8 Per-Group Dynamic Quantization, Group Size = 32"):

1. split each row into groups of 32 consecutive elements along K;
2. take the group's largest magnitude (amax);
3. derive the group's scale from amax and the element format's largest
   value, with an all-zero group mapped to scale 1 (section V item 4);
4. divide by the scale and clip to the format's range;
5. round to the element format.

Readings where the page leaves a step open:

* Scale.  The listing divides amax by the FP8 maximum; section III.3.2 says
  the scale is a power of two (an exponent).  Both hold, with no overflow
  (section V item 4), when amax / Qmax is rounded UP to a power of two:
  the scale exponent e is the smallest integer with amax <= Qmax * 2**e,
  clamped to [-127, 127] (the E8M0 range).  amax == 0 gives e = 0.
* Rounding: nearest, ties to even (the listing's cast to float8_e4m3fn
  rounds that way); the same rule is used for E2M1.
* The element value x * 2**-e is formed exactly (a power-of-two scaling).
* Clipping to +-Qmax is kept as in the listing; under the scale rule above
  it never changes a value.

FP4 codes are packed two per byte, element 2j in bits 3:0 and element 2j+1
in bits 7:4; scales are one byte per (row, block), row-major.
"""

import numpy as np

from . import formats as F

BLOCK = 32


def scale_exponent(amax, qmax):
    """Smallest integer e with amax <= qmax * 2**e, clamped to [-127, 127];
    amax == 0 -> 0.  Comparisons use exact power-of-two products."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    a = amax[nz]
    guess = np.ceil(np.log2(a / qmax)).astype(np.int64)
    # exact fix-up of the floating-point guess
    too_small = a > np.ldexp(qmax, guess)
    guess = guess + too_small
    too_big = a <= np.ldexp(qmax, guess - 1)
    guess = guess - too_big
    assert np.all(a <= np.ldexp(qmax, guess))
    assert np.all(a > np.ldexp(qmax, guess - 1))
    e[nz] = guess
    return np.clip(e, -127, 127)


def quantize_mx(x_bits, fmt):
    """Quantize BF16 rows [rows, K] (uint16 bit patterns), K % 32 == 0.

    Returns (codes, scales): codes uint8 [rows, K], one element code per
    byte (unpacked), and scale bytes uint8 [rows, K/32] (E8M0)."""
    spec = F.FORMATS[fmt]
    x = F.bf16_to_f64(x_bits)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize_mx: expected [rows, K] with K % 32 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_mx: non-finite input")
    rows, K = x.shape
    g = x.reshape(rows, K // BLOCK, BLOCK)  # step 1: groups of 32
    amax = np.abs(g).max(axis=-1)  # step 2
    e = scale_exponent(amax, spec["qmax"])  # step 3 (power-of-two scale)
    v = np.ldexp(g, -e[..., None])  # step 4: exact division by 2**e
    v = np.clip(v, -spec["qmax"], spec["qmax"])
    codes = spec["encode"](v)  # step 5
    return codes.reshape(rows, K).astype(np.uint8), (e + 127).astype(np.uint8)


def dequantize_mx(codes, scales, fmt):
    """codes [rows, K] (unpacked) and scales [rows, K/32] -> float64."""
    spec = F.FORMATS[fmt]
    codes = np.asarray(codes)
    rows, K = codes.shape
    vals = spec["decode"](codes).reshape(rows, K // BLOCK, BLOCK)
    s = F.e8m0_decode(scales)[..., None]
    return (vals * s).reshape(rows, K)


def pack_fp4(codes):
    """[rows, K] 4-bit codes -> [rows, K/2] bytes, even element low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_fp4(packed):
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def storage_codes(codes, fmt):
    """Codes in the byte layout the library stores (FP4 packed, FP8 as is)."""
    return pack_fp4(codes) if fmt == F.FMT_MXFP4 else np.asarray(codes, np.uint8)


def quantize_dequantize(x_bits, fmt):
    """deq(Q(x)) as float64."""
    c, s = quantize_mx(x_bits, fmt)
    return dequantize_mx(c, s, fmt)
