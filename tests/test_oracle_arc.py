"""Pins for oracle/arc.py: the hand-worked example, the exact linearity
identity, channel selection by brute force, S = 0 reduction."""

from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from oracle import arc as A
from synthetic import workloads as W
from tests import _golden as gold


def worked_inputs():
    a = np.zeros((1, 64))
    a[0, 0], a[0, 5], a[0, 40], a[0, 41] = 6.0, 0.75, 1.25, -2.5
    w = np.ones((2, 64))
    w[0, 1::2] = 2.0
    return F.f64_to_bf16(a), F.f64_to_bf16(w)


def test_worked_example():
    g = gold.keyed("arc_worked.txt")
    a, w = worked_inputs()
    idx = A.select_outlier_channels(a, 32)
    assert idx.tolist() == [int(v) for v in g["idx"]]
    ac, as_ = A.augment_activations(a, idx)
    assert as_[0, 2] == int(g["residual_scale_byte"][0])
    assert ac[0, 64:68].tolist() == [int(v) for v in g["residual_codes"]]
    wc, ws = A.augment_weights(w, idx)
    y_arc = G.gemm_mx(ac, as_, wc, ws, F.FMT_MXFP4)
    assert y_arc[0].tolist() == g["y_arc"]
    pc, ps = Q.quantize_mx(a, F.FMT_MXFP4)
    qc, qs = Q.quantize_mx(w, F.FMT_MXFP4)
    assert G.gemm_mx(pc, ps, qc, qs, F.FMT_MXFP4)[0].tolist() == g["y_plain"]


def test_linearity_identity_exact():
    """Y_arc = deq(P) deq(Q(W))^T + deq(R) deq(Q(W[:, idx]))^T, exactly."""
    rng = np.random.default_rng(8)
    a = F.f64_to_bf16(rng.standard_t(3, (3, 96)) * np.where(rng.random(96) < 0.1, 20, 1))
    w = F.f64_to_bf16(rng.normal(0, 0.02, (2, 96)))
    idx = A.select_outlier_channels(a, 32)
    y_arc = A.gemm_arc(a, w, idx)
    P = Q.quantize_dequantize(a, F.FMT_MXFP4)
    R = Q.quantize_dequantize(A.residual_bits(a, idx), F.FMT_MXFP4)
    WQ = Q.quantize_dequantize(w, F.FMT_MXFP4)
    WD = Q.quantize_dequantize(np.ascontiguousarray(w[:, idx]), F.FMT_MXFP4)
    e1 = G.exact_matmul(P, WQ)
    e2 = G.exact_matmul(R, WD)
    for m in range(3):
        for n in range(2):
            assert Fraction(float(y_arc[m, n])) == e1[m][n] + e2[m][n]


def test_selection_brute_force():
    rng = np.random.default_rng(6)
    a = F.f64_to_bf16(rng.standard_normal((16, 128)).round(1))  # many ties
    idx = A.select_outlier_channels(a, 64)
    x = F.bf16_to_f64(a)
    amax = [max(abs(x[m, k]) for m in range(16)) for k in range(128)]
    want = sorted(range(128), key=lambda k: (-amax[k], k))[:64]
    assert idx.tolist() == want


def test_s_zero_reduces_to_plain():
    d = W.c1_gemm_mxfp4(M=8, K=128, N=8)
    idx = np.zeros(0, np.int32)
    ac, as_ = A.augment_activations(d["a"], idx)
    pc, ps = Q.quantize_mx(d["a"], F.FMT_MXFP4)
    assert np.array_equal(ac, pc) and np.array_equal(as_, ps)


def test_representable_channels_give_zero_residual():
    a = np.zeros((2, 64))
    a[:, :32] = 1.0  # on the grid
    a[0, 40] = 3.0
    ab = F.f64_to_bf16(a)
    idx = np.arange(32, dtype=np.int32)
    ac, as_ = A.augment_activations(ab, idx)
    assert np.all(ac[:, 64:] == 0) and np.all(as_[:, 2] == 127)


def test_arc_beats_plain_on_outlier_activations():
    d = W.c3_arc(M=128, K=512, N=64, n_outliers=8)
    idx = A.select_outlier_channels(d["a"], 32)
    e_arc, e_plain = A.arc_errors(d["a"], d["w"], idx)
    assert e_arc < e_plain
