"""GPU parity of the fused ARC front end (rq_arc_frontend) and of
rq_rmsnorm: bit-exact codes and scales against the oracle wherever both
sides see the same BF16 inputs (no RMSNorm; rows whose RMSNorm is exact;
the oracle fed the GPU's own normalized rows), RMSNorm within one BF16 step
of the float64 oracle, and the config-3 augmented GEMM built on the front
end on sampled rows."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import arc as A
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from synthetic import workloads as W
from tests.gpu_util import bf16_ulp_dist, check_f32, dev, dev_bf16, host, host_bits, log

pytestmark = pytest.mark.gpu

FMTS = [(L.RQ_MXFP4, F.FMT_MXFP4), (L.RQ_MXFP8, F.FMT_MXFP8)]
MODES = [(L.RQ_APPEND_RESIDUAL, "residual"), (L.RQ_APPEND_COPY, "copy")]


def outlier_rows(rng, rows, K):
    x = rng.standard_t(3, (rows, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 20.0
    return F.f64_to_bf16(x)


def closed_form_rows(rng, rows, K):
    """Mean square 4: each 16-channel group holds ten +-1 and six +-3."""
    out = []
    for _ in range(rows):
        g = np.array([1.0] * 10 + [3.0] * 6)
        r = np.concatenate([rng.permutation(g) for _ in range(K // 16)])
        out.append(r * rng.choice([-1.0, 1.0], K))
    return F.f64_to_bf16(np.array(out))


def gpu_frontend(h_bits, perm, S, fmt, append, rmsnorm, eps=1e-6):
    c, s = api.arc_frontend(dev_bf16(h_bits), dev(np.asarray(perm, np.int32)), S, fmt, append, rmsnorm, eps)
    return host(c), host(s)


def expect(h_bits, perm, S, ofmt, mode, rmsnorm, eps=1e-6):
    c, s = A.frontend(h_bits, perm, S, ofmt, mode, rmsnorm, eps)
    return Q.storage_codes(c, ofmt), s


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("append,mode", MODES)
@pytest.mark.parametrize("rows,K,S", [(37, 4096, 128), (5, 96, 32), (3, 64, 64), (3, 16384, 256), (4, 8192, 32),
                                      (2501, 128, 32)])
def test_without_rmsnorm_bit_exact(fmt, ofmt, append, mode, rows, K, S):
    """Every row length class (one to eight chunks per thread), several rows
    per workgroup with a ragged last one (2501 rows), S from one block to K."""
    rng = np.random.default_rng(rows + K + S)
    h = outlier_rows(rng, rows, K)
    for perm in (A.reorder_permutation(h), rng.permutation(K)):
        c, s = gpu_frontend(h, perm, S, fmt, append, False)
        ec, es = expect(h, perm, S, ofmt, mode, False)
        assert np.array_equal(s, es) and np.array_equal(c, ec)
    c, s = gpu_frontend(h, np.arange(K), 0, fmt, L.RQ_APPEND_NONE, False)
    pc, ps = Q.quantize_mx(h, ofmt)
    assert np.array_equal(c, Q.storage_codes(pc, ofmt)) and np.array_equal(s, ps)
    log(f"front end without RMSNorm fmt={ofmt} {mode} rows={rows} K={K} S={S}: bit-exact")


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("append,mode", MODES)
def test_without_rmsnorm_extreme_block_exponents(fmt, ofmt, append, mode):
    """Every 32-channel group scaled by 2^u, u uniform over the BF16 range
    (subnormal to near the largest finite value), so primary blocks and
    residuals cover the clamped and subnormal scale bytes."""
    rng = np.random.default_rng(25)
    K = 1024
    x = rng.standard_normal((16, K)) * np.repeat(2.0 ** rng.integers(-140, 120, (16, K // 32)), 32, axis=1)
    h = F.f64_to_bf16(x)
    # move whole groups (and shuffle within each), so blocks keep one scale
    perm = (rng.permutation(K // 32)[:, None] * 32 + rng.permutation(32)[None, :]).ravel()
    c, s = gpu_frontend(h, perm, 256, fmt, append, False)
    ec, es = expect(h, perm, 256, ofmt, mode, False)
    assert es.min() <= 2 and es.max() >= 230  # the scale range is covered
    assert np.array_equal(s, es) and np.array_equal(c, ec)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("append,mode", MODES)
def test_closed_form_rmsnorm_rows_bit_exact(fmt, ofmt, append, mode):
    rng = np.random.default_rng(21)
    h = closed_form_rows(rng, 9, 512)
    perm = rng.permutation(512)
    c, s = gpu_frontend(h, perm, 64, fmt, append, True, 0.0)
    ec, es = expect(h, perm, 64, ofmt, mode, True, 0.0)
    assert np.array_equal(s, es) and np.array_equal(c, ec)


def test_rmsnorm_against_oracle():
    rng = np.random.default_rng(22)
    h = outlier_rows(rng, 300, 2048)
    n = host_bits(api.rmsnorm(dev_bf16(h), 1e-6))
    d = bf16_ulp_dist(n, A.rmsnorm_bits(h, 1e-6))
    log(f"rq_rmsnorm: {int((d > 0).sum())} of {d.size} elements one BF16 step from the float64 oracle")
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3
    e = closed_form_rows(rng, 4, 256)
    assert np.array_equal(host_bits(api.rmsnorm(dev_bf16(e), 0.0)), A.rmsnorm_bits(e, 0.0))


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_rmsnorm_inside_equals_rq_rmsnorm(fmt, ofmt):
    """The front end's normalized values are rq_rmsnorm's: fed the GPU's
    normalized rows, the oracle (without RMSNorm) gives the same codes."""
    rng = np.random.default_rng(23)
    h = outlier_rows(rng, 64, 4096)
    n = host_bits(api.rmsnorm(dev_bf16(h), 1e-6))
    perm = A.reorder_permutation(n)
    for append, mode in MODES:
        c, s = gpu_frontend(h, perm, 128, fmt, append, True)
        ec, es = expect(n, perm, 128, ofmt, mode, False)
        assert np.array_equal(s, es) and np.array_equal(c, ec)


def test_config3_front_end_gemm_sampled():
    """Config 3 through the front end: calibrate the channel order on the
    GPU-normalized activations (device amax + host sort), A' and W' from
    rq_arc_frontend, one MXFP4 GEMM over K + S; sampled rows against the
    oracle, and the error against the BF16 product of the normalized rows
    compared with plain MXFP4."""
    d = W.c3_arc(N=512)
    S, K = 128, 4096
    h = dev_bf16(d["a"])
    n = api.rmsnorm(h, 1e-6)
    perm = api.reorder_permutation(n)
    n_host = host_bits(n)
    assert np.array_equal(host(perm), A.reorder_permutation(n_host))
    ac, as_ = api.arc_frontend(h, perm, S)
    wc, ws = api.arc_frontend(dev_bf16(d["w"]), perm, S, append=L.RQ_APPEND_COPY, rmsnorm=False)
    y = host(api.gemm(L.RQ_MXFP4, ac, as_, wc, ws, K + S, L.RQ_OUT_F32))
    rows = np.union1d(np.random.default_rng(24).choice(4096, 24, replace=False), [0, 4095])
    pa, pas = A.frontend(n_host[rows], host(perm), S, F.FMT_MXFP4, "residual", False)
    pw, pws = A.frontend(d["w"], host(perm), S, F.FMT_MXFP4, "copy", False)
    ref = G.gemm_mx(pa, pas, pw, pws, F.FMT_MXFP4)
    bound = G.abs_bound(Q.dequantize_mx(pa, pas, F.FMT_MXFP4), Q.dequantize_mx(pw, pws, F.FMT_MXFP4))
    check_f32(y[rows], ref, bound, "config-3 front-end GEMM")
    exact = G.gemm_bf16(n_host[rows], d["w"])
    qa, qas = Q.quantize_mx(n_host[rows], F.FMT_MXFP4)
    qw, qws = Q.quantize_mx(d["w"], F.FMT_MXFP4)
    e_plain = G.rel_frobenius(G.gemm_mx(qa, qas, qw, qws, F.FMT_MXFP4), exact)
    e_front = G.rel_frobenius(ref, exact)
    log(f"config 3 on normalized rows: fused ARC front end {e_front:.4f} vs plain MXFP4 {e_plain:.4f}")
    assert e_front < e_plain
