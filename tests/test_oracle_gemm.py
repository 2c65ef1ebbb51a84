"""Pins for oracle/gemm.py: exact rational brute force, special cases."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G


def random_codes(rng, rows, K, fmt):
    if fmt == F.FMT_MXFP4:
        return rng.integers(0, 16, (rows, K)).astype(np.uint8)
    c = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return c


@pytest.mark.parametrize("fmt", [F.FMT_MXFP4, F.FMT_MXFP8])
def test_mx_gemm_matches_exact_rationals(fmt):
    rng = np.random.default_rng(21)
    M, N, K = 3, 5, 96  # non-square, 3 blocks: a transposed operand fails
    ac, wc = random_codes(rng, M, K, fmt), random_codes(rng, N, K, fmt)
    as_ = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    ws = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    y = G.gemm_mx(ac, as_, wc, ws, fmt)
    # independent brute force straight from codes: sum over blocks of
    # 2**(ea+ew-254) * sum_k qa*qw, in exact rationals
    dec = F.FORMATS[fmt]["decode"]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for b in range(K // 32):
                part = Fraction(0)
                pmag = Fraction(0)
                for k in range(32 * b, 32 * b + 32):
                    t = Fraction(float(dec(ac[m, k]))) * Fraction(float(dec(wc[n, k])))
                    part += t
                    pmag += abs(t)
                sc = Fraction(2) ** (int(as_[m, b]) + int(ws[n, b]) - 254)
                tot += part * sc
                mag += pmag * sc
            if fmt == F.FMT_MXFP4:
                # <= 4 significant bits per product, few binades: exact in fp64
                assert Fraction(float(y[m, n])) == tot, (m, n)
            else:
                # E4M3 spans 2**-9..448 per element, so the fp64 sum may
                # round; it stays within K fp64 roundings of the exact sum
                assert abs(Fraction(float(y[m, n])) - tot) <= K * Fraction(2) ** -52 * mag, (m, n)


def test_identity_weights_select_columns():
    rng = np.random.default_rng(2)
    K = 64
    ac = random_codes(rng, 4, K, F.FMT_MXFP4)
    as_ = rng.integers(120, 135, (4, 2)).astype(np.uint8)
    # W row n has a single 1.0 (code 0x2) at column n, scale byte 127
    wc = np.zeros((K, K), dtype=np.uint8)
    wc[np.arange(K), np.arange(K)] = 0x2
    ws = np.full((K, 2), 127, dtype=np.uint8)
    y = G.gemm_mx(ac, as_, wc, ws, F.FMT_MXFP4)
    assert np.array_equal(y, Q.dequantize_mx(ac, as_, F.FMT_MXFP4))


def test_single_block_hand_dot():
    # K = 32: a = [1, 2, -3, 0.5, 0...] (codes 2, 4, D, 1), scale 2**1;
    #         w = [6, 1, 1, -4, 0...] (codes 7, 2, 2, E), scale 2**-2.
    # sum = 6 + 2 - 3 - 2 = 3;  y = 3 * 2**1 * 2**-2 = 1.5
    ac = np.zeros((1, 32), np.uint8)
    ac[0, :4] = [0x2, 0x4, 0xD, 0x1]
    wc = np.zeros((1, 32), np.uint8)
    wc[0, :4] = [0x7, 0x2, 0x2, 0xE]
    y = G.gemm_mx(ac, np.array([[128]], np.uint8), wc, np.array([[125]], np.uint8), F.FMT_MXFP4)
    assert y[0, 0] == 1.5


def test_bf16_gemm_exact_small():
    rng = np.random.default_rng(4)
    a = F.f64_to_bf16(rng.standard_normal((2, 40)))
    w = F.f64_to_bf16(rng.standard_normal((3, 40)))
    y = G.gemm_bf16(a, w)
    ex = G.exact_matmul(F.bf16_to_f64(a), F.bf16_to_f64(w))
    for m in range(2):
        for n in range(3):
            assert Fraction(float(y[m, n])) == ex[m][n]


def test_tolerance_helpers():
    a = np.array([[1.0, -2.0]])
    w = np.array([[3.0, 4.0], [-1.0, 0.5]])
    assert G.abs_bound(a, w).tolist() == [[11.0, 2.0]]
    assert G.rel_frobenius(np.array([3.0, 4.0]), np.array([3.0, 4.0])) == 0.0
    assert G.rel_frobenius(np.array([0.0, 0.0]), np.array([3.0, 4.0])) == 1.0
