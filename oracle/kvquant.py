"""FP8 per-token-head-tile quantize-on-write with float32 scales.

Oracle (test infrastructure).  Follows the Day-0 page (Day 0 LLM Inference
Support, section III.3.3 "KV Cache: FP8 Per-Token-Head-Tile Quantization,
Tile Size = 128", and the per-group listing of section V, which the page
says the KV variant follows with a token x head x 128 grouping):

1. group each (token, head) vector into tiles of 128 consecutive elements;
2. amax per tile;
3. scale = amax / 448, or 1 for an all-zero tile;
4. q = x / scale, clipped to +-448;
5. cast to E4M3FN (nearest, ties to even).

Reading: unlike the power-of-two MX scale, this scale is the plain quotient
amax / 448, kept as float32; steps 3 and 4 are float32 operations (one
IEEE rounding each, as a float32 tensor pipeline performs them), because
the float result decides the integer code and both sides must decide it in
the same precision.
"""

import numpy as np

from . import formats as F

TILE = 128
FP8_MAX = np.float32(448.0)


def quantize_kv(x_bits, tile=TILE):
    """x BF16 bits [T, H, D] (D % tile == 0) -> (codes uint8 [T, H, D],
    scales float32 [T, H, D/tile])."""
    x32 = F.bf16_to_f64(x_bits).astype(np.float32)  # exact
    T, H, D = x32.shape
    if D % tile:
        raise ValueError("head dim must be a multiple of the tile")
    g = x32.reshape(T, H, D // tile, tile)
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax > 0, amax / FP8_MAX, np.float32(1.0)).astype(np.float32)
    q = (g / scale[..., None]).astype(np.float32)
    q = np.clip(q, -FP8_MAX, FP8_MAX)
    codes = F.e4m3_encode(q.astype(np.float64))
    return codes.reshape(T, H, D).astype(np.uint8), scale


def dequantize_kv(codes, scales, tile=TILE):
    T, H, D = codes.shape
    v = F.e4m3_decode(codes).reshape(T, H, D // tile, tile)
    return (v * scales.astype(np.float64)[..., None]).reshape(T, H, D)
