"""Number formats: BF16, E2M1 (FP4), E4M3FN (FP8), E8M0 (shared scale).

Oracle (test infrastructure).  Written from the format definitions:

* E2M1 is the element type the ARCQuant page names for its 4-bit blocks
  (ARCQuant: Boosting NVFP4 Quantization with Augmented Residual Channels,
  technical summary, "Methodologie").  Its eight magnitudes are
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} (sign bit, 2 exponent bits with bias 1,
  1 mantissa bit; code 1 is the subnormal 0.5), as in the OCP Microscaling
  (MX) v1.0 element tables.
* E4M3FN is the FP8 type of the per-group pseudo-code on the Day-0 page
  (Day 0 LLM Inference Support: Hierarchical Quantization and Memory Access
  Optimization Practices, section V, per-group dynamic quantization
  listing): 4 exponent bits with bias 7, 3 mantissa bits, largest finite
  value 448, no infinities, 0x7F/0xFF are NaN.
* E8M0 is the power-of-two shared scale (same page, section III.3.2: the
  scaling factor is an exponent): a byte b stands for 2**(b - 127); 0xFF is
  NaN.
* BF16 keeps the float32 exponent and an 8-bit significand; conversions
  round to nearest, ties to even.

Encoders are written as a plain search: the nearest finite magnitude of the
table, and on an exact tie the candidate with the even code.  Negative
inputs keep their sign bit even when they round to zero (as torch's
float8_e4m3fn cast does), so -0 encodes as 0x8 (E2M1) or 0x80 (E4M3).
"""

import numpy as np

FMT_MXFP4 = "mxfp4"
FMT_MXFP8 = "mxfp8"

# ---------------------------------------------------------------- BF16 ----


def bf16_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """float64 -> BF16 bit patterns, one rounding: nearest, ties to even.

    The BF16 grid in the binade [2**(ex-1), 2**ex) has step 2**(ex-8); below
    the smallest normal (2**-126) the step stays 2**-133 (subnormals).
    Scaling by a power of two is exact in float64, so ``rint`` of the scaled
    value is the single correct rounding.  Values that round past the
    largest finite BF16 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("f64_to_bf16: non-finite input")
    _, ex = np.frexp(x)
    step = np.maximum(ex, -125) - 8
    y = np.ldexp(np.rint(np.ldexp(x, -step)), step)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)  # exact: y has <= 8 significant bits
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def f32_to_bf16(x32):
    """float32 -> BF16 bits (nearest, ties to even)."""
    return f64_to_bf16(np.asarray(x32, dtype=np.float32).astype(np.float64))


# ---------------------------------------------------------------- E2M1 ----

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_SIGN_BIT = 3
E2M1_MAX = 6.0


def e2m1_decode(codes):
    """4-bit E2M1 codes (0..15) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c >> E2M1_SIGN_BIT) & 1, -mag, mag)


# ---------------------------------------------------------------- E4M3 ----


def _e4m3_magnitude(code):
    """Magnitude of a 7-bit E4M3FN code from the format definition."""
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return m * 2.0 ** -9  # subnormal: m/8 * 2**(1-7)
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Finite magnitudes, indexed by code 0x00..0x7E (0x7F is NaN).
E4M3_MAGNITUDES = np.array([_e4m3_magnitude(c) for c in range(0x7F)])
E4M3_SIGN_BIT = 7
E4M3_MAX = 448.0
assert E4M3_MAGNITUDES[-1] == E4M3_MAX


def e4m3_decode(codes):
    """8-bit E4M3FN codes -> float64 (NaN codes raise)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("e4m3_decode: NaN code")
    mag = E4M3_MAGNITUDES[c & 0x7F]
    return np.where((c >> E4M3_SIGN_BIT) & 1, -mag, mag)


# ---------------------------------------------------------------- E8M0 ----


def e8m0_decode(b):
    """E8M0 scale bytes -> float64 2**(b-127) (0xFF is NaN and raises)."""
    b = np.asarray(b).astype(np.int64)
    if np.any(b == 0xFF):
        raise ValueError("e8m0_decode: NaN scale")
    return np.ldexp(1.0, b - 127)


# ------------------------------------------------------ nearest-even ----


def encode_nearest_even(v, magnitudes, sign_bit):
    """Round each v to the nearest finite magnitude of the table; on an
    exact tie take the even code.  Returns integer codes with the sign bit
    set for negative inputs (including -0)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v).ravel()
    mags = np.asarray(magnitudes, dtype=np.float64)
    # Midpoints between neighbouring magnitudes: a value strictly between
    # two midpoints has one nearest magnitude; a value on a midpoint ties.
    mids = 0.5 * (mags[:-1] + mags[1:])
    idx = np.searchsorted(mids, a, side="left")  # a <= mids[idx]
    on_mid = np.zeros(a.shape, dtype=bool)
    inb = idx < len(mids)
    on_mid[inb] = a[inb] == mids[idx[inb]]
    # a tie between codes idx and idx+1: keep the even one
    tie_up = on_mid & (idx % 2 == 1)
    codes = idx + tie_up.astype(np.int64)
    if np.any(a > mags[-1]):
        raise ValueError("encode_nearest_even: value beyond the format maximum")
    codes = codes.reshape(v.shape)
    return codes | (np.signbit(v).astype(np.int64) << sign_bit)


def e2m1_encode(v):
    return encode_nearest_even(v, E2M1_MAGNITUDES, E2M1_SIGN_BIT)


def e4m3_encode(v):
    return encode_nearest_even(v, E4M3_MAGNITUDES, E4M3_SIGN_BIT)


FORMATS = {
    FMT_MXFP4: dict(qmax=E2M1_MAX, encode=e2m1_encode, decode=e2m1_decode, bits=4),
    FMT_MXFP8: dict(qmax=E4M3_MAX, encode=e4m3_encode, decode=e4m3_decode, bits=8),
}
