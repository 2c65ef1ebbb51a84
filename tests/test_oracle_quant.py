"""Pins for oracle/quant.py: scale rule, element encode, packing, round trip.

Pinned against hand-derived worked blocks (tests/golden/), exact rational
brute force of the scale rule, exhaustive BF16 sweeps, and torch running the
Day-0 page's per-group listing with the power-of-two scale."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q
from tests import _golden as gold
from tests.test_oracle_formats import all_finite_bf16

QMAX = {F.FMT_MXFP4: 6, F.FMT_MXFP8: 448}


def block_bits(values):
    row = np.zeros(32, dtype=np.float64)
    for i, (v, _) in values.items():
        row[i] = v
    bits = F.f64_to_bf16(row)
    assert np.array_equal(F.bf16_to_f64(bits), row), "fixture value not BF16-exact"
    # keep -0 entries
    for i, (v, _) in values.items():
        if v == 0 and np.signbit(v):
            bits[i] = 0x8000
    return bits[None, :]


@pytest.mark.parametrize("blk", gold.mx_blocks(), ids=lambda b: b[0])
def test_worked_blocks(blk):
    name, fmt, scale_byte, values = blk
    codes, scales = Q.quantize_mx(block_bits(values), fmt)
    assert scales.shape == (1, 1) and scales[0, 0] == scale_byte, (name, scales)
    want = np.zeros(32, dtype=np.uint8)
    for i, (_, c) in values.items():
        want[i] = c
    assert np.array_equal(codes[0], want), (name, codes[0], want)


def test_scale_rule_exact_brute_force():
    """For random blocks: Qmax*2**(e-1) < amax <= Qmax*2**e in exact
    rationals, unless the exponent is clamped at -127."""
    rng = np.random.default_rng(11)
    for fmt in (F.FMT_MXFP4, F.FMT_MXFP8):
        for scale in (1e-38, 1e-20, 1e-3, 1.0, 1e3, 1e30):
            x = F.f64_to_bf16(rng.standard_normal((8, 64)) * scale)
            _, s = Q.quantize_mx(x, fmt)
            amax = np.abs(F.bf16_to_f64(x)).reshape(8, 2, 32).max(-1)
            for a, b in zip(amax.ravel(), s.ravel()):
                e = int(b) - 127
                A = Fraction(float(a))
                assert A <= QMAX[fmt] * Fraction(2) ** e
                if e > -127:
                    assert A > QMAX[fmt] * Fraction(2) ** (e - 1)


@pytest.mark.parametrize("fmt", [F.FMT_MXFP4, F.FMT_MXFP8])
def test_exhaustive_bf16_as_block_max(fmt):
    """Every finite BF16 x as the only nonzero of a block: its scale obeys
    the rule and its code is the grid point nearest to x / 2**e, found by
    brute force over the signed code table."""
    bits = all_finite_bf16()
    x = np.zeros((bits.size, 32), dtype=np.uint16)
    x[:, 0] = bits
    codes, scales = Q.quantize_mx(x, fmt)
    xv = F.bf16_to_f64(bits)
    e = scales[:, 0].astype(np.int64) - 127
    a = np.abs(xv)
    nz = a > 0
    assert np.all(a[nz] <= QMAX[fmt] * np.ldexp(1.0, e[nz]))
    unclamped = nz & (e > -127)
    assert np.all(a[unclamped] > QMAX[fmt] * np.ldexp(1.0, e[unclamped] - 1))
    assert np.all(e[~nz] == 0)
    ncode = 16 if fmt == F.FMT_MXFP4 else 256
    table = np.array([F.FORMATS[fmt]["decode"](c) if (fmt == F.FMT_MXFP4 or (c & 0x7F) != 0x7F) else np.nan
                      for c in range(ncode)])
    v = np.ldexp(xv, -e)
    d = np.abs(v[:, None] - table[None, :])
    d[:, np.isnan(table)] = np.inf
    best = d.min(axis=1)
    got = codes[:, 0].astype(np.int64)
    assert np.array_equal(d[np.arange(len(got)), got], best)
    # among exact ties the even code wins (both signs of zero are distance 0:
    # the code must carry the input's sign)
    tie = (np.sum(d == best[:, None], axis=1) > 1) & (best > 0)
    assert np.all(got[tie] % 2 == 0)
    assert np.array_equal(np.signbit(xv), (got >> (3 if fmt == F.FMT_MXFP4 else 7)) == 1)
    # unused elements are +0
    assert np.all(codes[:, 1:] == 0)


@pytest.mark.parametrize("fmt", [F.FMT_MXFP4, F.FMT_MXFP8])
def test_round_trip_on_representable_values(fmt):
    """Blocks g * 2**e0 with g on the grid and max |g| in (Qmax/2, Qmax]
    quantize back to exactly their codes and scale."""
    rng = np.random.default_rng(5)
    ncode = 8 if fmt == F.FMT_MXFP4 else 0x7F
    sb = 3 if fmt == F.FMT_MXFP4 else 7
    decode = F.FORMATS[fmt]["decode"]
    rows = 256
    mag = rng.integers(0, ncode, (rows, 32))
    top = rng.integers(6 if fmt == F.FMT_MXFP4 else 0x77, ncode, rows)  # max in (Qmax/2, Qmax]
    mag[np.arange(rows), rng.integers(0, 32, rows)] = top
    sign = rng.integers(0, 2, (rows, 32))
    sign[mag == 0] = 0
    codes_in = mag | (sign << sb)
    e0 = rng.integers(-100, 100, rows)
    x = decode(codes_in) * np.ldexp(1.0, e0)[:, None]
    xb = F.f64_to_bf16(x)
    assert np.array_equal(F.bf16_to_f64(xb), x)
    codes, scales = Q.quantize_mx(xb, fmt)
    assert np.array_equal(codes, codes_in.astype(np.uint8))
    assert np.array_equal(scales[:, 0], (e0 + 127).astype(np.uint8))


@pytest.mark.parametrize("fmt", [F.FMT_MXFP4, F.FMT_MXFP8])
def test_idempotent(fmt):
    rng = np.random.default_rng(9)
    x = F.f64_to_bf16(rng.standard_t(3, (64, 128)))
    d1 = Q.quantize_dequantize(x, fmt)
    d2 = Q.quantize_dequantize(F.f64_to_bf16(d1), fmt)
    assert np.array_equal(d1, d2)


def test_pack_nibble_order():
    c = np.array([[0x1, 0x2, 0xF, 0x8]], dtype=np.uint8)
    p = Q.pack_fp4(c)
    assert p.tolist() == [[0x21, 0x8F]]
    assert np.array_equal(Q.unpack_fp4(p), c)


def test_mxfp8_matches_day0_listing_run_in_torch():
    """Torch runs the Day-0 per-group listing (amax, divide, clip, cast to
    float8_e4m3fn) with the scale rounded up to a power of two; codes must
    agree with the oracle's."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((512, 256)) * np.exp(rng.uniform(-20, 20, (512, 1)))
    xb = F.f64_to_bf16(x)
    codes, scales = Q.quantize_mx(xb, F.FMT_MXFP8)
    g = torch.from_numpy(F.bf16_to_f64(xb)).reshape(-1, 32)
    scale = torch.from_numpy(np.ldexp(1.0, scales.astype(np.int64).ravel() - 127)).reshape(-1, 1)
    q = (g / scale).clamp(-448.0, 448.0).to(torch.float32).to(torch.float8_e4m3fn)
    ref = q.view(torch.uint8).numpy().reshape(512, 256)
    assert np.array_equal(codes, ref)


def test_zero_and_negative_zero_blocks():
    x = np.zeros((2, 32), dtype=np.uint16)
    x[1, 3] = 0x8000
    for fmt in (F.FMT_MXFP4, F.FMT_MXFP8):
        codes, scales = Q.quantize_mx(x, fmt)
        assert np.all(scales == 127)
        assert codes[1, 3] == (0x8 if fmt == F.FMT_MXFP4 else 0x80)
        assert np.count_nonzero(codes) == 1
