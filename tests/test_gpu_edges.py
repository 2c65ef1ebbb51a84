"""Degenerate and boundary cases across the entry points, on the GPU:
empty inputs leave the outputs untouched, one-element and one-block
shapes, every token flagged or none, the longest schedule, and S = K for
the ARC front end -- each against the oracle or the property that defines
the case."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import arc as A
from oracle import formats as F
from oracle import gemm as G
from oracle import gemv as V
from oracle import quant as Q
from oracle import ramp as R
from synthetic import workloads as W
from tests.gpu_util import check_f32, dev, dev_bf16, host, host_bits, log

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def test_gemm_empty_m_or_n_leaves_output():
    a = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    s = torch.full((4, 2), 127, dtype=torch.uint8, device="cuda")
    y = torch.full((4, 4), SENTINEL, dtype=torch.int16, device="cuda")
    for M, N in ((0, 4), (4, 0)):
        L.rq_gemm(L.RQ_MXFP8, a, s, a, s, M, N, 64, L.RQ_OUT_BF16, y)
    assert np.all(host(y) == SENTINEL)


@pytest.mark.parametrize("fmt,ofmt", [(L.RQ_MXFP4, F.FMT_MXFP4), (L.RQ_MXFP8, F.FMT_MXFP8)])
def test_gemm_one_output_one_block(fmt, ofmt):
    rng = np.random.default_rng(31)
    a = F.f64_to_bf16(rng.standard_normal((1, 32)))
    w = F.f64_to_bf16(rng.standard_normal((1, 32)))
    ac, as_ = Q.quantize_mx(a, ofmt)
    wc, ws = Q.quantize_mx(w, ofmt)
    y = host(api.gemm(fmt, dev(Q.storage_codes(ac, ofmt)), dev(as_), dev(Q.storage_codes(wc, ofmt)), dev(ws), 32,
                      L.RQ_OUT_F32))
    ref = G.gemm_mx(ac, as_, wc, ws, ofmt)
    check_f32(y, ref, G.abs_bound(Q.dequantize_mx(ac, as_, ofmt), Q.dequantize_mx(wc, ws, ofmt)), "1x1x32")


def test_front_end_empty_rows_and_s_equal_k():
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    c, s = api.arc_frontend(x, torch.arange(64, dtype=torch.int32, device="cuda"), 32)
    assert c.shape == (0, 48) and s.shape == (0, 3)  # K + S = 96 elements: 48 bytes of codes, 3 scales
    rng = np.random.default_rng(32)
    h = F.f64_to_bf16(rng.standard_t(3, (6, 64)))
    perm = rng.permutation(64)
    c, s = api.arc_frontend(dev_bf16(h), dev(perm.astype(np.int32)), 64, rmsnorm=False)  # every channel gets a residual
    ec, es = A.frontend(h, perm, 64, F.FMT_MXFP4, "residual", False)
    assert np.array_equal(host(s), es) and np.array_equal(host(c), Q.storage_codes(ec, F.FMT_MXFP4))


def gemv_case(N, K, B, flags, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sc = (rng.random((N, K // 32)) * 0.01 + 0.001).astype(np.float16)
    x = F.f64_to_bf16(rng.standard_normal((B, K)))
    planes = api.pack_nibble_planes(dev(w), dev(sc.view(np.int16)))
    fl = dev(np.asarray(flags, np.uint8))
    y = host_bits(api.gemv_nibble_escalate(dev_bf16(x), N, planes, fl, L.RQ_BOTH))
    return x, w, sc, y


def test_gemv_one_row_one_token_and_all_or_no_tokens_flagged():
    # N = 1, B = 1, flagged: the full 8-bit product
    x, w, sc, y = gemv_case(1, 64, 1, [1], 33)
    want = V.gemv_nibble_escalate(x, w, sc, np.array([1], np.uint8))
    assert np.max(np.abs(F.bf16_to_f64(y) - F.bf16_to_f64(want))) <= 2.0 ** -7 * np.abs(F.bf16_to_f64(want)).max()
    for flags in ([0] * 16, [1] * 16):
        x, w, sc, y = gemv_case(200, 96, 16, flags, 34)
        want = V.gemv_nibble_escalate(x, w, sc, np.array(flags, np.uint8))
        bound = V.abs_bound(x, w if flags[0] else V.split_nibbles(w)[0].astype(np.int64) * 16, sc)
        err = np.abs(F.bf16_to_f64(y) - F.bf16_to_f64(want))
        assert np.all(err <= 1e-3 * bound + np.abs(F.bf16_to_f64(want)) * 2.0 ** -7), flags[0]
        log(f"GEMV with {sum(flags)} of 16 tokens flagged: max err {err.max():.3e}")


def test_recurrent_prefill_longest_schedule_and_empty():
    """64 steps (the longest) on a tiny block equals the oracle's 64-step
    trajectory within the recurrence tolerance; zero rows is a no-op."""
    d = W.c4_ramp(S=8, D=64, F=128)
    w1d, w2d = dev_bf16(d["w1"]), dev_bf16(d["w2"])
    w1q, w2q = api.quantize(w1d, L.RQ_MXFP4), api.quantize(w2d, L.RQ_MXFP4)
    sched = 0x0F0F0F0F0F0F0F0F
    h = dev_bf16(d["h0"])
    api.recurrent_prefill(h, w1d, w2d, w1q, w2q, L.RQ_MXFP4, sched, 64)
    o = R.ramp_prefill(d["h0"], d["w1"], d["w2"], sched, 64, F.FMT_MXFP4)
    o_bf = R.ramp_prefill(d["h0"], d["w1"], d["w2"], 0, 64, F.FMT_MXFP4)
    err = np.linalg.norm(F.bf16_to_f64(host_bits(h)) - F.bf16_to_f64(o)) / np.linalg.norm(F.bf16_to_f64(o))
    # the same rule as the 8-step schedules: a tenth of the schedule's own
    # distance from the all-BF16 trajectory
    tol = max(1e-3, 0.1 * R.hidden_relative_error(o, o_bf))
    log(f"64-step schedule: gpu-vs-oracle {err:.3e} (tol {tol:.2e})")
    assert err <= tol
    e = torch.zeros((0, 64), dtype=torch.int16, device="cuda")
    api.recurrent_prefill(e, w1d, w2d, w1q, w2q, L.RQ_MXFP4, sched, 4)
    assert e.numel() == 0


def test_kv_quantize_empty_and_gate_two_logits():
    x = torch.zeros((0, 2, 128), dtype=torch.int16, device="cuda")
    c, s = api.kv_quantize(x)
    assert c.numel() == 0 and s.numel() == 0
    z = F.f64_to_bf16(np.array([[1.0, 1.0], [5.0, -5.0]]))
    flags, stats = api.escalation_gate(dev_bf16(z), 0.5, 0.1)
    st = host(stats)
    assert np.allclose(st[0], [np.log(2.0), 0.0], atol=1e-5)  # a tie: entropy ln 2, gap 0
    assert host(flags).tolist() == [1, 0]


def test_grouped_gemv_one_problem_all_flagged():
    rng = np.random.default_rng(35)
    N, K, B = 130, 64, 16
    w = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sc = (rng.random((N, K // 32)) * 0.01 + 0.001).astype(np.float16)
    x = dev_bf16(F.f64_to_bf16(rng.standard_normal((B, K))))
    planes = api.pack_nibble_planes(dev(w), dev(sc.view(np.int16)))
    fl = dev(np.ones(B, np.uint8))
    want = host_bits(api.gemv_nibble_escalate(x, N, planes, fl, L.RQ_BOTH, split=False))
    y = torch.zeros((B, N), dtype=torch.bfloat16, device="cuda")
    api.gemv_nibble_escalate_grouped(api.gemv_group([(x, planes, y)]), B, fl, L.RQ_BOTH)
    assert np.array_equal(host_bits(y), want)


@pytest.mark.parametrize("a_exp,w_exp", [((10, 13), (200, 231)), ((240, 247), (20, 51))])
def test_mxfp8_exact_at_extreme_block_exponents(a_exp, w_exp):
    """RQ_MXFP8 dequantizes to BF16 in registers: exact down to block
    exponent -117 (scale byte 10: every E4M3 value, subnormals included,
    is then a normal BF16) and up to the largest exponent a BF16 block
    produces (119, byte 246); tiny activations meet huge weights and the
    reverse, so the products come back into the FP32 range."""
    rng = np.random.default_rng(a_exp[0])
    M, N, K = 64, 64, 256
    ac = rng.integers(0, 256, (M, K)).astype(np.uint8)
    ac[(ac & 0x7F) == 0x7F] = 0x7E
    wc = rng.integers(0, 256, (N, K)).astype(np.uint8)
    wc[(wc & 0x7F) == 0x7F] = 0x7E
    as_ = rng.integers(*a_exp, (M, K // 32)).astype(np.uint8)
    ws = rng.integers(*w_exp, (N, K // 32)).astype(np.uint8)
    log(f"MXFP8 extreme block exponents a {a_exp} w {w_exp}")
    y = host(api.gemm(L.RQ_MXFP8, dev(ac), dev(as_), dev(wc), dev(ws), K, L.RQ_OUT_F32))
    ref = G.gemm_mx(ac, as_, wc, ws, F.FMT_MXFP8)
    bound = G.abs_bound(Q.dequantize_mx(ac, as_, F.FMT_MXFP8), Q.dequantize_mx(wc, ws, F.FMT_MXFP8))
    check_f32(y, ref, bound, "extreme exponents")
