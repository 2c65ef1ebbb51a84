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


# ---------------------------------------------------------------- front end --

def test_frontend_worked_example():
    g = gold.keyed("arc_frontend_worked.txt")
    h = np.zeros((1, 64))
    h[0, 0], h[0, 1] = 3.0, 4.0
    hb = F.f64_to_bf16(h)
    n = A.rmsnorm_bits(hb, 1e-6)
    assert F.bf16_to_f64(n)[0, :2].tolist() == g["n_bf16"]
    perm = A.reorder_permutation(n)
    assert perm[:4].tolist() == [int(v) for v in g["perm_head"]]
    ac, as_ = A.frontend(hb, perm, 32, eps=1e-6)
    assert ac[0, :3].tolist() == [int(v) for v in g["primary_codes"]]
    assert as_[0, :2].tolist() == [int(v) for v in g["primary_scale_bytes"]]
    assert ac[0, 64:67].tolist() == [int(v) for v in g["residual_codes"]]
    assert as_[0, 2] == int(g["residual_scale_byte"][0])
    cc, cs = A.frontend(hb, perm, 32, append="copy", eps=1e-6)
    assert cc[0, 64:67].tolist() == [int(v) for v in g["copy_codes"]]
    assert cs[0, 2] == int(g["copy_scale_byte"][0])
    w = F.f64_to_bf16(np.ones((1, 64)))
    wc, ws = A.frontend(w, perm, 32, append="copy", rmsnorm=False)
    y_arc = G.gemm_mx(ac, as_, wc, ws, F.FMT_MXFP4)
    pc, ps = A.frontend(hb, perm, 0, eps=1e-6)
    qc, qs = A.frontend(w, perm, 0, append="copy", rmsnorm=False)
    assert y_arc[0, 0] == g["y_arc"][0]
    assert G.gemm_mx(pc, ps, qc, qs, F.FMT_MXFP4)[0, 0] == g["y_plain"][0]
    assert float(F.bf16_to_f64(n)[0] @ np.ones(64)) == g["y_exact"][0]


def test_frontend_applies_the_permutation_not_its_inverse():
    """Channels 0, 1, 2 hold 1, 4, 2 (no RMSNorm): the amax order is 1, 2, 0,
    so positions 0..2 hold 4, 2, 1 -- block amax 4, e = 0 -- with E2M1 codes
    0x6, 0x4, 0x2 (the inverse order would give 0x4, 0x2, 0x6)."""
    x = np.zeros((1, 64))
    x[0, :3] = [1.0, 4.0, 2.0]
    xb = F.f64_to_bf16(x)
    perm = A.reorder_permutation(xb)
    assert perm[:3].tolist() == [1, 2, 0]
    c, s = A.frontend(xb, perm, 0, rmsnorm=False)
    assert c[0, :3].tolist() == [0x6, 0x4, 0x2] and s[0, 0] == 127


def test_reorder_permutation_brute_force():
    rng = np.random.default_rng(11)
    x = F.f64_to_bf16(rng.standard_normal((8, 96)).round(1))  # many ties
    perm = A.reorder_permutation(x)
    v = F.bf16_to_f64(x)
    amax = [max(abs(v[m, k]) for m in range(8)) for k in range(96)]
    assert perm.tolist() == sorted(range(96), key=lambda k: (-amax[k], k))
    assert sorted(perm.tolist()) == list(range(96))


def test_frontend_reduces_to_block_quantization():
    """S = 0 with the identity order: the front end is RMSNorm then the
    standard block quantization (and the quantization alone without it)."""
    rng = np.random.default_rng(12)
    h = F.f64_to_bf16(rng.standard_t(3, (5, 128)))
    ident = np.arange(128)
    for fmt in (F.FMT_MXFP4, F.FMT_MXFP8):
        c, s = A.frontend(h, ident, 0, fmt, rmsnorm=False)
        pc, ps = Q.quantize_mx(h, fmt)
        assert np.array_equal(c, pc) and np.array_equal(s, ps)
        c, s = A.frontend(h, ident, 0, fmt, eps=1e-6)
        pc, ps = Q.quantize_mx(F.f64_to_bf16(F.bf16_to_f64(h) / np.sqrt(
            (F.bf16_to_f64(h) ** 2).mean(axis=1, keepdims=True) + 1e-6)), fmt)
        assert np.array_equal(c, pc) and np.array_equal(s, ps)


def test_frontend_rmsnorm_closed_form_rows():
    """Rows whose mean square is 4: RMSNorm with eps = 0 halves every value
    exactly.  Each group of 16 channels holds ten +-1 and six +-3 (sum of
    squares 64)."""
    rng = np.random.default_rng(13)
    rows = []
    for _ in range(4):
        g = np.array([1.0] * 10 + [3.0] * 6)
        r = np.concatenate([rng.permutation(g) for _ in range(8)])
        rows.append(r * rng.choice([-1.0, 1.0], 128))
    h = np.array(rows)
    n = A.rmsnorm_bits(F.f64_to_bf16(h), 0.0)
    assert np.array_equal(F.bf16_to_f64(n), h / 2)


def test_frontend_grid_values_exact_for_any_order():
    """Values on the E2M1 grid (times a power of two per row) quantize
    exactly in any block arrangement, so for every permutation the
    augmented product equals the exact product and the residual is zero."""
    rng = np.random.default_rng(14)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(grid, (3, 96)) * rng.choice([-1, 1], (3, 96)) * 2.0 ** rng.integers(-3, 4, (3, 1))
    w = rng.choice(grid, (2, 96)) * rng.choice([-1, 1], (2, 96))
    xb, wb = F.f64_to_bf16(x), F.f64_to_bf16(w)
    for perm in (np.arange(96), rng.permutation(96), A.reorder_permutation(xb)):
        ac, as_ = A.frontend(xb, perm, 32, rmsnorm=False)
        wc, ws = A.frontend(wb, perm, 32, append="copy", rmsnorm=False)
        assert np.all(ac[:, 96:] == 0)
        y = G.gemm_mx(ac[:, :96], as_[:, :3], wc[:, :96], ws[:, :3], F.FMT_MXFP4)
        assert np.array_equal(y, x @ w.T)


def test_frontend_residual_never_increases_the_error():
    """For the S outlier positions: |x - deq(P) - deq(R)| <= |x - deq(P)|
    (0 is on every grid and the scale rule never clips), and the appended
    product is the exact sum of the primary and residual products."""
    rng = np.random.default_rng(15)
    h = F.f64_to_bf16(rng.standard_t(3, (4, 128)) * np.where(rng.random(128) < 0.1, 20, 1))
    w = F.f64_to_bf16(rng.normal(0, 0.02, (2, 128)))
    n = A.rmsnorm_bits(h, 1e-6)
    perm = A.reorder_permutation(n)
    ac, as_ = A.frontend(h, perm, 32, eps=1e-6)
    x = F.bf16_to_f64(n)[:, perm]
    dp = Q.dequantize_mx(ac[:, :128], as_[:, :4], F.FMT_MXFP4)
    dr = Q.dequantize_mx(ac[:, 128:], as_[:, 4:], F.FMT_MXFP4)
    assert np.all(np.abs(x[:, :32] - dp[:, :32] - dr) <= np.abs(x[:, :32] - dp[:, :32]))
    wc, ws = A.frontend(w, perm, 32, append="copy", rmsnorm=False)
    y = G.gemm_mx(ac, as_, wc, ws, F.FMT_MXFP4)
    dw = Q.dequantize_mx(wc, ws, F.FMT_MXFP4)
    e1 = G.exact_matmul(dp, dw[:, :128])
    e2 = G.exact_matmul(dr, dw[:, 128:])
    for m in range(4):
        for j in range(2):
            assert Fraction(float(y[m, j])) == e1[m][j] + e2[m][j]
