"""GPU parity of rq_gemm_arc: the hand-worked example, small shapes against
the oracle, and the full 4096^3 (K' = 4224) workload on sampled rows, with
the ARC-versus-plain error ordering."""

import numpy as np
import pytest

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from oracle import arc as A
from synthetic import workloads as W
from tests import _golden as gold
from tests.gpu_util import check_f32, dev, dev_bf16, host, log, rel_fro

pytestmark = pytest.mark.gpu


def gpu_arc(a_bits, w_bits, S, out=L.RQ_OUT_F32):
    a = dev_bf16(a_bits)
    idx = api.select_channels(api.channel_amax(a), S)
    idx_d = dev(idx.numpy())
    wc, ws = api.quantize(dev_bf16(w_bits), L.RQ_MXFP4, idx_d, L.RQ_APPEND_COPY)
    y = api.gemm_arc(a, idx_d, wc, ws, out)
    return y, idx.numpy(), (wc, ws)


def test_worked_example():
    g = gold.keyed("arc_worked.txt")
    a = np.zeros((1, 64))
    a[0, 0], a[0, 5], a[0, 40], a[0, 41] = 6.0, 0.75, 1.25, -2.5
    w = np.ones((2, 64))
    w[0, 1::2] = 2.0
    y, idx, _ = gpu_arc(F.f64_to_bf16(a), F.f64_to_bf16(w), 32)
    assert idx.tolist() == [int(v) for v in g["idx"]]
    assert host(y)[0].tolist() == g["y_arc"]


def test_small_against_oracle():
    d = W.c3_arc(M=256, K=512, N=192, n_outliers=16)
    for S in (32, 64):
        y, idx, (wc, ws) = gpu_arc(d["a"], d["w"], S)
        assert np.array_equal(idx, A.select_outlier_channels(d["a"], S))
        owc, ows = A.augment_weights(d["w"], idx)
        assert np.array_equal(host(wc), Q.pack_fp4(owc)) and np.array_equal(host(ws), ows)
        ac, as_ = A.augment_activations(d["a"], idx)
        ref = G.gemm_mx(ac, as_, owc, ows, F.FMT_MXFP4)
        bound = G.abs_bound(Q.dequantize_mx(ac, as_, F.FMT_MXFP4), Q.dequantize_mx(owc, ows, F.FMT_MXFP4))
        log(f"ARC S={S} rel fro {check_f32(host(y), ref, bound, 'ARC small'):.2e}")


def test_config3_full_size_sampled_and_error_ordering():
    d = W.c3_arc()
    y, idx, (wc, ws) = gpu_arc(d["a"], d["w"], 128)
    assert np.array_equal(idx, A.select_outlier_channels(d["a"], 128))
    rows = np.sort(np.random.default_rng(5).choice(4096, 32, replace=False))
    ys = host(y)[rows]
    owc, ows = A.augment_weights(d["w"], idx)
    assert np.array_equal(host(wc)[:64], Q.pack_fp4(owc[:64]))
    ac, as_ = A.augment_activations(d["a"][rows], idx)
    da, dw = Q.dequantize_mx(ac, as_, F.FMT_MXFP4), Q.dequantize_mx(owc, ows, F.FMT_MXFP4)
    ref = G.matmul_f64(da, dw)
    log(f"config-3 ARC rel fro {check_f32(ys, ref, G.abs_bound(da, dw), 'config-3 ARC'):.2e}")
    # reported property: ARC is closer than plain MXFP4 to the BF16-operand product
    pc, ps = api.quantize(dev_bf16(d["a"]), L.RQ_MXFP4)
    qc, qs = api.quantize(dev_bf16(d["w"]), L.RQ_MXFP4)
    yp = host(api.gemm(L.RQ_MXFP4, pc, ps, qc, qs, 4096, L.RQ_OUT_F32))[rows]
    exact = G.matmul_f64(F.bf16_to_f64(d["a"][rows]), F.bf16_to_f64(d["w"]))
    e_arc, e_plain = rel_fro(ys, exact), rel_fro(yp, exact)
    log(f"config-3 error vs BF16 operands: ARC {e_arc:.4e}  plain {e_plain:.4e}")
    assert e_arc < e_plain
