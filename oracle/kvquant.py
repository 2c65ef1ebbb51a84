"""FP8 per-token-head-tile quantize-on-write with float32 scales.

Oracle (test infrastructure).  Follows the Day-0 page (Day 0 LLM Inference
Support, section III.3.3, "KV Cache: FP8 Per-Token-Head-Tile Quantization,
Tile Size = 128"): within each token and head, every run of 128 consecutive
elements shares one scaling factor, and the page says the per-group recipe
of section V carries over with that grouping.  Written out from the
mathematics of that recipe:

* a tile's scaling factor is its largest magnitude divided by the largest
  E4M3FN value, 448; a tile of zeros gets the factor 1 (nothing to divide);
* every element is divided by its tile's factor, limited to [-448, 448] and
  rounded to the nearest E4M3FN value (ties to the even code).

Reading: the factor is the plain quotient (not a power of two) and is kept
in float32, and the element division is a float32 operation; both decide
the integer code, so the GPU makes them in the same precision.
"""

import numpy as np

from . import formats as F

TILE = 128
E4M3_LARGEST = np.float32(448.0)


def tile_factor(tile_max):
    """float32 largest magnitudes -> float32 scaling factors (1 where 0)."""
    tile_max = np.asarray(tile_max, dtype=np.float32)
    safe = np.where(tile_max > 0, tile_max, np.float32(448.0))
    return np.where(tile_max > 0, np.divide(safe, E4M3_LARGEST, dtype=np.float32), np.float32(1.0))


def encode_tiles(tiles, factors):
    """tiles float32 [..., TILE], factors float32 [...] -> E4M3FN codes."""
    ratio = np.divide(tiles, factors[..., None], dtype=np.float32)
    limited = np.minimum(np.maximum(ratio, -E4M3_LARGEST), E4M3_LARGEST)
    return F.e4m3_encode(limited.astype(np.float64))


def quantize_kv(x_bits, tile=TILE):
    """x BF16 bits [T, H, D] (D % tile == 0) -> (codes uint8 [T, H, D],
    scales float32 [T, H, D/tile])."""
    vals = F.bf16_to_f64(x_bits).astype(np.float32)  # every BF16 value is a float32
    T, H, D = vals.shape
    if D % tile:
        raise ValueError("head dim must be a multiple of the tile")
    tiles = vals.reshape(T, H, D // tile, tile)
    factors = tile_factor(np.max(np.abs(tiles), axis=-1))
    codes = encode_tiles(tiles, factors)
    return codes.reshape(T, H, D).astype(np.uint8), factors.astype(np.float32)


def dequantize_kv(codes, scales, tile=TILE):
    T, H, D = codes.shape
    v = F.e4m3_decode(codes).reshape(T, H, D // tile, tile)
    return (v * scales.astype(np.float64)[..., None]).reshape(T, H, D)
