"""Pins for oracle/gemv.py: exhaustive nibble split, the hand-worked GEMV,
multiples-of-16 reduction, exact rationals, and oracle/gate.py."""

from fractions import Fraction

import numpy as np
import scipy.stats

from oracle import formats as F
from oracle import gemv as V
from oracle import gate as GT
from tests import _golden as gold


def test_nibble_split_exhaustive():
    w = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    hi, lo = V.split_nibbles(w)
    assert hi.min() == -8 and hi.max() == 7 and lo.min() == 0 and lo.max() == 15
    assert np.array_equal(16 * hi.astype(np.int64) + lo, w.astype(np.int64))
    back = ((hi.astype(np.int64) << 4) | lo).astype(np.uint8).view(np.int8)
    assert np.array_equal(back, w)
    # the low weight is w with its low nibble cleared
    assert np.array_equal(16 * hi.astype(np.int64), w.astype(np.int64) & ~15)


def worked():
    w = np.zeros((2, 32), np.int8)
    w[0, :6] = [127, -128, -1, 16, 15, -17]
    w[1, :] = 16
    s = np.array([[0.5], [0.25]], dtype=np.float16)
    x = np.zeros((2, 32))
    x[0, :6] = 1.0
    x[1, 0], x[1, 5] = 2.0, -1.0
    return w, s, F.f64_to_bf16(x)


def test_worked_gemv():
    g = gold.keyed("gemv_worked.txt")
    w, s, x = worked()
    assert F.f64_to_bf16(V.low_pass(x, w, s)).view(np.uint16).tolist() == \
        F.f64_to_bf16(np.array(g["y_low"]).reshape(2, 2)).tolist()
    full = F.bf16_to_f64(F.f64_to_bf16(V.full_pass(x, w, s)))
    assert full.ravel().tolist() == g["y_full"]
    mixed = F.bf16_to_f64(V.gemv_nibble_escalate(x, w, s, np.array([0, 1])))
    assert mixed.ravel().tolist() == g["y_mixed"]
    hi, lo = V.pack_planes(w)
    assert hi[0, :3].tolist() == [int(v) for v in g["hi_plane_row0"]]
    assert lo[0, :3].tolist() == [int(v) for v in g["lo_plane_row0"]]


def test_abs_bound_hand_values():
    """sum_k |x_k w_k s| on the worked example, by hand: row 0 of W is
    [127, -128, -1, 16, 15, -17] at scale 0.5 (low weights 16 hi =
    [112, -128, -16, 16, 0, -32]); row 1 is all 16 at scale 0.25."""
    w, s, x = worked()
    full = V.abs_bound(x, w, s)
    assert full.tolist() == [[(127 + 128 + 1 + 16 + 15 + 17) * 0.5, 6 * 4.0], [(2 * 127 + 17) * 0.5, 3 * 4.0]]
    hi, _ = V.split_nibbles(w)
    low = V.abs_bound(x, 16 * hi.astype(np.int64), s)
    assert low.tolist() == [[(112 + 128 + 16 + 16 + 0 + 32) * 0.5, 24.0], [(2 * 112 + 32) * 0.5, 12.0]]
    # a sign flip of x or w leaves it unchanged; it bounds |y| of every sign pattern
    assert np.array_equal(V.abs_bound(F.f64_to_bf16(-F.bf16_to_f64(x)), -w.astype(np.int64), s), full)
    assert np.all(np.abs(V.full_pass(x, w, s)) <= full)


def test_multiples_of_16_low_equals_full():
    rng = np.random.default_rng(0)
    w = (rng.integers(-8, 8, (40, 64)) * 16).astype(np.int8)
    s = rng.uniform(0.001, 0.01, (40, 2)).astype(np.float16)
    x = F.f64_to_bf16(rng.standard_normal((16, 64)))
    assert np.array_equal(V.low_pass(x, w, s), V.full_pass(x, w, s))


def test_gemv_exact_rationals():
    rng = np.random.default_rng(1)
    w = rng.integers(-128, 128, (3, 64)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, (3, 2)).astype(np.float16)
    x = F.f64_to_bf16(rng.standard_normal((2, 64)))
    y = V.full_pass(x, w, s)
    xv = F.bf16_to_f64(x)
    for t in range(2):
        for n in range(3):
            tot = sum(Fraction(float(xv[t, k])) * int(w[n, k]) * Fraction(float(s[n, k // 32]))
                      for k in range(64))
            assert Fraction(float(y[t, n])) == tot


def test_only_flagged_rows_change():
    rng = np.random.default_rng(2)
    w = rng.integers(-128, 128, (32, 64)).astype(np.int8)
    s = rng.uniform(0.001, 0.01, (32, 2)).astype(np.float16)
    x = F.f64_to_bf16(rng.standard_normal((4, 64)))
    flags = np.array([0, 1, 0, 1], np.uint8)
    y = V.gemv_nibble_escalate(x, w, s, flags)
    lo = F.f64_to_bf16(V.low_pass(x, w, s))
    fu = F.f64_to_bf16(V.full_pass(x, w, s))
    assert np.array_equal(y[[0, 2]], lo[[0, 2]]) and np.array_equal(y[[1, 3]], fu[[1, 3]])


def test_gate_closed_forms_and_scipy():
    V_ = 1000
    uniform = np.zeros((1, V_))
    peaked = np.zeros((1, V_))
    peaked[0, 7] = 60.0
    tie = np.zeros((1, V_)) - 30
    tie[0, 3] = tie[0, 9] = 10.0
    logits = F.f64_to_bf16(np.concatenate([uniform, peaked, tie]))
    h, gap = GT.softmax_stats(logits)
    assert abs(h[0] - np.log(V_)) < 1e-12 and gap[0] == 0
    assert h[1] < 1e-20 and abs(gap[1] - 1) < 1e-20
    assert gap[2] == 0
    rng = np.random.default_rng(3)
    z = F.f64_to_bf16(rng.standard_normal((4, 500)) * 3)
    zv = F.bf16_to_f64(z)
    p = np.exp(zv - zv.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    h2, _ = GT.softmax_stats(z)
    assert np.allclose(h2, scipy.stats.entropy(p, axis=1), rtol=1e-12)
    f = GT.escalation_flags(logits, tau=1.0, delta=0.1)
    assert f.tolist() == [1, 0, 1]
