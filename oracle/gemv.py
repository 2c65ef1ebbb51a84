"""Decode GEMV on 8-bit weights read through their top nibble, with 8-bit
recompute of flagged tokens.

Oracle (test infrastructure).  Follows the escalation article (Escalating
Weight Precision Only When Decoding Becomes Uncertain, the setup paragraph):
weights are stored with 8 bits, a first low-precision pass decodes with
their top four bits, and a step whose output looks uncertain is computed
again with the full 8-bit weights.

Readings:

* "Top four bits" of a signed int8 w is hi = w >> 4 (arithmetic shift,
  -8..7); the low-precision weight is 16 * hi, i.e. w with its low nibble
  cleared.  No midpoint correction is added.
* lo = w & 15 (0..15), so w = 16 * hi + lo exactly.
* Each 32-element block of a weight row along K has an FP16 scale s; the
  dequantized weights are 16 * hi * s (low) and w * s (full).
* A flagged token's row of y is replaced by the full-precision result (the
  step is recomputed, not blended).
* y = x . W^T is accumulated in float64 and rounded once to BF16.

Plane layout (the library's storage, also produced here for parity): the
hi and lo nibbles are each packed two per byte along K, element 2j in bits
3:0 and 2j+1 in bits 7:4; hi is stored as its 4-bit two's complement.
"""

import numpy as np

from . import formats as F

BLOCK = 32


def split_nibbles(w):
    """int8 [N, K] -> (hi int8 in -8..7, lo uint8 in 0..15)."""
    w = np.asarray(w, dtype=np.int8)
    hi = (w >> 4).astype(np.int8)
    lo = (w & 15).astype(np.uint8)
    return hi, lo


def pack_planes(w):
    """int8 [N, K] -> (hi_plane, lo_plane), each uint8 [N, K/2]."""
    hi, lo = split_nibbles(w)
    h4 = hi.astype(np.uint8) & 0xF
    hi_plane = h4[:, 0::2] | (h4[:, 1::2] << 4)
    lo_plane = lo[:, 0::2] | (lo[:, 1::2] << 4)
    return hi_plane.astype(np.uint8), lo_plane.astype(np.uint8)


def _scaled(wint, scales_f16):
    """int weights [N, K] times per-32 FP16 scales [N, K/32] -> float64."""
    N, K = wint.shape
    s = np.asarray(scales_f16, dtype=np.float16).astype(np.float64)
    return (wint.astype(np.float64).reshape(N, K // BLOCK, BLOCK) * s[..., None]).reshape(N, K)


def gemv_f64(x_bits, wint, scales_f16):
    """x [B, K] BF16 bits, integer weights [N, K], scales -> float64 [B, N]."""
    x = F.bf16_to_f64(x_bits)
    return x @ _scaled(wint, scales_f16).T


def low_pass(x_bits, w, scales_f16):
    hi, _ = split_nibbles(w)
    return gemv_f64(x_bits, 16 * hi.astype(np.int64), scales_f16)


def full_pass(x_bits, w, scales_f16):
    return gemv_f64(x_bits, np.asarray(w, dtype=np.int64), scales_f16)


def gemv_nibble_escalate(x_bits, w, scales_f16, flags):
    """BF16 [B, N]: low-pass rows, flagged rows replaced by the 8-bit result."""
    y = low_pass(x_bits, w, scales_f16)
    flags = np.asarray(flags).astype(bool)
    if flags.any():
        y_full = full_pass(x_bits[flags], w, scales_f16)
        y[flags] = y_full
    return F.f64_to_bf16(y)


def abs_bound(x_bits, wint, scales_f16):
    """sum_k |x_k * w_k| per output, for the per-element tolerance."""
    x = np.abs(F.bf16_to_f64(x_bits))
    return x @ np.abs(_scaled(np.asarray(wint, np.int64), scales_f16)).T
