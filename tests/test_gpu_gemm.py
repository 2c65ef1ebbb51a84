"""GPU parity of rq_gemm: a single-tile probe that pins the scaled-MFMA
operand/scale/output layouts, multi-tile and ragged shapes, the workload
shapes at full size (sampled rows where the float64 oracle would be slow),
BF16 output = RNE(FP32 output), determinism."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from oracle import quant as Q
from oracle import gemm as G
from synthetic import workloads as W
from tests.gpu_util import REL_FRO, check_bf16, check_f32, dev, dev_bf16, host, host_bits, log, rel_fro

pytestmark = pytest.mark.gpu

MX = [(L.RQ_MXFP4, F.FMT_MXFP4), (L.RQ_MXFP8, F.FMT_MXFP8)]


def random_codes(rng, rows, K, ofmt):
    if ofmt == F.FMT_MXFP4:
        return rng.integers(0, 16, (rows, K)).astype(np.uint8)
    c = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def run_mx(fmt, ofmt, ac, as_, wc, ws, out=L.RQ_OUT_F32):
    K = ac.shape[1]
    a = dev(Q.storage_codes(ac, ofmt))
    w = dev(Q.storage_codes(wc, ofmt))
    y = api.gemm(fmt, a, dev(as_), w, dev(ws), K, out)
    return host(y.float()) if out == L.RQ_OUT_F32 else host_bits(y)


@pytest.mark.parametrize("fmt,ofmt", MX)
def test_single_tile_probe(fmt, ofmt):
    """One 32 x 32 output, K = 64: distinct codes and per-(row, block) scales."""
    rng = np.random.default_rng(1)
    ac, wc = random_codes(rng, 32, 64, ofmt), random_codes(rng, 32, 64, ofmt)
    # block exponents within +-9 of 1.0 keep the two-block sums below exact in FP32
    as_ = rng.integers(122, 132, (32, 2)).astype(np.uint8)
    ws = rng.integers(122, 132, (32, 2)).astype(np.uint8)
    log(f"single-tile probe fmt={ofmt}")
    y = run_mx(fmt, ofmt, ac, as_, wc, ws)
    ref = G.gemm_mx(ac, as_, wc, ws, ofmt)
    bound = G.abs_bound(Q.dequantize_mx(ac, as_, ofmt), Q.dequantize_mx(wc, ws, ofmt))
    check_f32(y, ref, bound, "single tile")
    # scale association alone: every code 1.0, so y = 32 * sum_b 2^(sa+sw-254)
    one = np.full((32, 64), 0x2 if ofmt == F.FMT_MXFP4 else 0x38, np.uint8)
    y1 = run_mx(fmt, ofmt, one, as_, one, ws)
    want = 32.0 * (np.ldexp(1.0, as_[:, None, 0].astype(int) + ws[None, :, 0].astype(int) - 254)
                   + np.ldexp(1.0, as_[:, None, 1].astype(int) + ws[None, :, 1].astype(int) - 254))
    assert np.array_equal(y1, want), f"scale/layout mismatch, first bad {np.argwhere(y1 != want)[:4]}"


@pytest.mark.parametrize("fmt,ofmt", MX)
@pytest.mark.parametrize("M,N,K", [(200, 130, 96), (257, 300, 4224), (1, 1, 32), (128, 128, 128)])
def test_multi_tile_ragged(fmt, ofmt, M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = F.f64_to_bf16(rng.standard_t(3, (M, K)))
    w = F.f64_to_bf16(rng.normal(0, 0.02, (N, K)))
    ac, as_ = Q.quantize_mx(a, ofmt)
    wc, ws = Q.quantize_mx(w, ofmt)
    log(f"gemm fmt={ofmt} M={M} N={N} K={K}")
    y = run_mx(fmt, ofmt, ac, as_, wc, ws)
    ref = G.gemm_mx(ac, as_, wc, ws, ofmt)
    bound = G.abs_bound(Q.dequantize_mx(ac, as_, ofmt), Q.dequantize_mx(wc, ws, ofmt))
    check_f32(y, ref, bound, "F32 output")
    yb = run_mx(fmt, ofmt, ac, as_, wc, ws, L.RQ_OUT_BF16)
    assert np.array_equal(yb, F.f32_to_bf16(y.astype(np.float32))), "BF16 output != RNE(F32 output)"
    check_bf16(yb, ref, bound, "BF16 output", k=K)


@pytest.mark.parametrize("fmt,ofmt", MX)
@pytest.mark.parametrize("M,N,K", [(512, 384, 512), (4096, 4096, 256), (300, 200, 1280)])
def test_scale_association_every_block(fmt, ofmt, M, N, K):
    """Every code 1.0 and a distinct scale per (row, block): y[m, n] =
    32 sum_b 2^(sa[m,b] + sw[n,b] - 254) exactly (a 10-bit exponent spread
    keeps every partial sum exact), for the 128 and 256 tile paths."""
    rng = np.random.default_rng(K + M)
    nb = K // 32
    as_ = rng.integers(125, 131, (M, nb)).astype(np.uint8)
    ws = rng.integers(125, 131, (N, nb)).astype(np.uint8)
    code = 0x2 if ofmt == F.FMT_MXFP4 else 0x38
    log(f"scale association fmt={ofmt} M={M} N={N} K={K}")
    y = run_mx(fmt, ofmt, np.full((M, K), code, np.uint8), as_, np.full((N, K), code, np.uint8), ws)
    want = 32.0 * (np.ldexp(1.0, as_.astype(int) - 127) @ np.ldexp(1.0, ws.astype(int) - 127).T)
    assert np.array_equal(y, want), f"scale/layout mismatch, first bad {np.argwhere(y != want)[:4]}"


@pytest.mark.parametrize("fmt,ofmt", MX + [(L.RQ_BF16, None)])
@pytest.mark.parametrize("M,N,K", [(4000, 4100, 384), (4096, 4096, 128), (3969, 4097, 1152), (4096, 4096, 160),
                                   (4096, 6100, 384), (4000, 5700, 1152)])
def test_large_tiles_ragged_sampled(fmt, ofmt, M, N, K):
    """Shapes with at least 256 tiles of 256 x 256 (the large-tile paths:
    256 x 256, and 256 x 192 for the last two, whose rounds it fills),
    ragged in M and N, K of one stage, an odd number of stages, a long tail
    and K ending in a partial stage (MXFP4 at 384 and 1152, BF16 at 160);
    the oracle runs on sampled rows that include the last one."""
    sampled_shape_check(fmt, ofmt, M, N, K, "large-tile")


def sampled_shape_check(fmt, ofmt, M, N, K, label):
    rng = np.random.default_rng(M + 3 * N + K)
    a = F.f64_to_bf16(rng.standard_t(3, (M, K)))
    w = F.f64_to_bf16(rng.normal(0, 0.02, (N, K)))
    rows = np.union1d(rng.choice(M, 24, replace=False), [0, M - 1])
    log(f"{label} gemm fmt={fmt} M={M} N={N} K={K}")
    if fmt == L.RQ_BF16:
        y = host(api.gemm(fmt, dev_bf16(a), None, dev_bf16(w), None, K, L.RQ_OUT_F32))[rows]
        da, dw = F.bf16_to_f64(a[rows]), F.bf16_to_f64(w)
        check_f32(y, G.matmul_f64(da, dw), G.abs_bound(da, dw), f"{label} BF16")
        return
    sampled_rows_check(fmt, ofmt, a, w, rows, f"{label} {ofmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt,ofmt", MX + [(L.RQ_BF16, None)])
@pytest.mark.parametrize("M,N,K", [(2048, 1024, 1056), (2049, 1000, 1024), (1000, 900, 544)])
def test_small_tile_boundary_sampled(fmt, ofmt, M, N, K):
    """Either side of the 64 x 64 rule (128 x 128 tiles for at most half
    the CUs): 2048 x 1024 makes exactly 128 such tiles (64 x 64 path, K
    ending in a partial stage), 2049 x 1000 makes 136 (128 x 128, three
    stages, ragged M and N), 1000 x 900 makes 64 (64 x 64, ragged)."""
    sampled_shape_check(fmt, ofmt, M, N, K, "tile-boundary")


@pytest.mark.parametrize("M,N,K", [(2049, 1000, 3072), (1100, 2100, 3200)])
def test_mxfp8_two_k_groups_sampled(M, N, K):
    """Exact MXFP8 shapes with 128 x 128 tiles for at most one per CU and K
    of at least 24 stages, whose workgroups sum even and odd slices in two
    groups of waves and add the second group's sums to the first's: ragged
    M and N (136 and 153 tiles), K of 24 and 25 stages; sampled rows against
    the oracle, and two runs bit for bit alike."""
    sampled_shape_check(L.RQ_MXFP8, F.FMT_MXFP8, M, N, K, "two-k-group")
    rng = np.random.default_rng(M + N + K)
    ac = dev(random_codes(rng, M, K, F.FMT_MXFP8))
    wc = dev(random_codes(rng, N, K, F.FMT_MXFP8))
    as_ = dev(rng.integers(118, 136, (M, K // 32)).astype(np.uint8))
    ws = dev(rng.integers(118, 136, (N, K // 32)).astype(np.uint8))
    y1 = host(api.gemm(L.RQ_MXFP8, ac, as_, wc, ws, K, L.RQ_OUT_F32))
    y2 = host(api.gemm(L.RQ_MXFP8, ac, as_, wc, ws, K, L.RQ_OUT_F32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("fmt,ofmt", MX + [(L.RQ_BF16, None)])
@pytest.mark.parametrize("M,N,K", [(4000, 2000, 4160), (4096, 2048, 5632), (3000, 1900, 2048)])
def test_tall_tiles_long_k_sampled(fmt, ofmt, M, N, K):
    """Shapes with more 128 x 128 tiles than CUs but at most 256 tiles of
    256 x 128, and K of at least 16 stages (the 256 x 128 path): ragged M
    and N, K ending in a partial stage (MXFP4 at 4160), the recurrent
    block's second GEMM; at 3000 x 1900 x 2048 MXFP8 and BF16 take the path
    and MXFP4 (8 stages) stays on 128 x 128 tiles."""
    sampled_shape_check(fmt, ofmt, M, N, K, "tall-tile")


@pytest.mark.parametrize("M,N,K", [(200, 130, 96), (129, 257, 512), (64, 64, 32)])
def test_bf16_gemm(M, N, K):
    rng = np.random.default_rng(M * N)
    a = F.f64_to_bf16(rng.standard_normal((M, K)))
    w = F.f64_to_bf16(rng.standard_normal((N, K)))
    log(f"bf16 gemm M={M} N={N} K={K}")
    y = host(api.gemm(L.RQ_BF16, dev_bf16(a), None, dev_bf16(w), None, K, L.RQ_OUT_F32))
    ref = G.gemm_bf16(a, w)
    bound = G.abs_bound(F.bf16_to_f64(a), F.bf16_to_f64(w))
    check_f32(y, ref, bound, "BF16 GEMM")
    yb = host_bits(api.gemm(L.RQ_BF16, dev_bf16(a), None, dev_bf16(w), None, K, L.RQ_OUT_BF16))
    assert np.array_equal(yb, F.f32_to_bf16(y.astype(np.float32)))


def quantize_on_gpu(bits, fmt):
    return api.quantize(dev_bf16(bits), fmt)


def test_config1_full():
    d = W.c1_gemm_mxfp4()
    ac, as_ = quantize_on_gpu(d["a"], L.RQ_MXFP4)
    wc, ws = quantize_on_gpu(d["w"], L.RQ_MXFP4)
    y = host(api.gemm(L.RQ_MXFP4, ac, as_, wc, ws, 1024, L.RQ_OUT_F32))
    oa, osa = Q.quantize_mx(d["a"], F.FMT_MXFP4)
    ow, osw = Q.quantize_mx(d["w"], F.FMT_MXFP4)
    ref = G.gemm_mx(oa, osa, ow, osw, F.FMT_MXFP4)
    bound = G.abs_bound(Q.dequantize_mx(oa, osa, F.FMT_MXFP4), Q.dequantize_mx(ow, osw, F.FMT_MXFP4))
    log(f"config-1 rel fro {check_f32(y, ref, bound, 'config 1'):.2e}")


def sampled_rows_check(fmt, ofmt, a_bits, w_bits, rows, what):
    """GPU quantize + GEMM at full size; oracle on the sampled rows only."""
    M, K = a_bits.shape
    ac, as_ = quantize_on_gpu(a_bits, fmt)
    wc, ws = quantize_on_gpu(w_bits, fmt)
    y = api.gemm(fmt, ac, as_, wc, ws, K, L.RQ_OUT_F32)
    yb = api.gemm(fmt, ac, as_, wc, ws, K, L.RQ_OUT_BF16)
    y = host(y)[rows]
    yb = host_bits(yb)[rows]
    oa, osa = Q.quantize_mx(a_bits[rows], ofmt)
    ow, osw = Q.quantize_mx(w_bits, ofmt)
    da, dw = Q.dequantize_mx(oa, osa, ofmt), Q.dequantize_mx(ow, osw, ofmt)
    ref = G.matmul_f64(da, dw)
    rf = check_f32(y, ref, G.abs_bound(da, dw), what)
    check_bf16(yb, ref, G.abs_bound(da, dw), what, k=K)
    log(f"{what}: rel fro {rf:.2e}")


def test_config2_linear_set_full_size_sampled():
    rng = np.random.default_rng(2)
    for i in range(7):
        d = W.c2_linear(i)
        rows = np.sort(rng.choice(4096, 48, replace=False))
        sampled_rows_check(L.RQ_MXFP8, F.FMT_MXFP8, d["a"], d["w"], rows, f"config-2 {d['name']}")


@pytest.mark.parametrize("gi", [0, 2])
def test_config2_stacked_group_equals_separate_linears(gi):
    """q/k/v (gate/up) on their shared input as one GEMM against the stacked
    weights (256 x 256 tiles) gives bit for bit the members' own GEMMs
    (128 x 128 tiles): per-row block scales make stacking commute with
    quantization, and every output's K order is the same in both tilings.
    Sampled rows of the stacked output are also checked against the oracle."""
    g = W.c2_layer()[gi]
    M, K = g["a"].shape
    ac, as_ = quantize_on_gpu(g["a"], L.RQ_MXFP8)
    wc, ws = quantize_on_gpu(g["w"], L.RQ_MXFP8)
    log(f"stacked {g['name']}: {M}x{g['w'].shape[0]}x{K}")
    y = host_bits(api.gemm(L.RQ_MXFP8, ac, as_, wc, ws, K, L.RQ_OUT_BF16))
    n0 = 0
    for name, n in zip(g["members"], g["Ns"]):
        ym = host_bits(api.gemm(L.RQ_MXFP8, ac, as_, wc[n0:n0 + n], ws[n0:n0 + n], K, L.RQ_OUT_BF16))
        assert np.array_equal(y[:, n0:n0 + n], ym), f"{name}: stacked != separate"
        n0 += n
    rows = np.sort(np.random.default_rng(gi).choice(M, 16, replace=False))
    oa, osa = Q.quantize_mx(g["a"][rows], F.FMT_MXFP8)
    ow, osw = Q.quantize_mx(g["w"], F.FMT_MXFP8)
    da, dw = Q.dequantize_mx(oa, osa, F.FMT_MXFP8), Q.dequantize_mx(ow, osw, F.FMT_MXFP8)
    check_bf16(y[rows], G.matmul_f64(da, dw), G.abs_bound(da, dw), g["name"], k=K)


def test_config3_plain_full_size_sampled():
    d = W.c3_arc()
    rows = np.sort(np.random.default_rng(3).choice(4096, 32, replace=False))
    sampled_rows_check(L.RQ_MXFP4, F.FMT_MXFP4, d["a"], d["w"], rows, "config-3 plain MXFP4 4096^3")


def test_config3_bf16_reference_sampled():
    d = W.c3_arc()
    rows = np.sort(np.random.default_rng(4).choice(4096, 32, replace=False))
    y = host(api.gemm(L.RQ_BF16, dev_bf16(d["a"]), None, dev_bf16(d["w"]), None, 4096, L.RQ_OUT_F32))[rows]
    a, w = F.bf16_to_f64(d["a"][rows]), F.bf16_to_f64(d["w"])
    log(f"config-3 BF16 rel fro {check_f32(y, G.matmul_f64(a, w), G.abs_bound(a, w), 'config-3 BF16'):.2e}")


@pytest.mark.parametrize("fmt", [L.RQ_MXFP4, L.RQ_MXFP8, L.RQ_BF16])
def test_deterministic(fmt):
    d = W.c2_linear(4, M=1024)
    if fmt == L.RQ_BF16:
        a, sa, w, sw = dev_bf16(d["a"]), None, dev_bf16(d["w"]), None
    else:
        a, sa = quantize_on_gpu(d["a"], fmt)
        w, sw = quantize_on_gpu(d["w"], fmt)
    y1 = host(api.gemm(fmt, a, sa, w, sw, 1024, L.RQ_OUT_F32))
    y2 = host(api.gemm(fmt, a, sa, w, sw, 1024, L.RQ_OUT_F32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_zero_operand_gives_zero():
    a = torch.zeros((70, 64), dtype=torch.uint8, device="cuda")
    s = torch.full((70, 4), 127, dtype=torch.uint8, device="cuda")
    w = torch.randint(0, 255, (50, 64), dtype=torch.uint8, device="cuda")
    ws = torch.full((50, 4), 127, dtype=torch.uint8, device="cuda")
    y = api.gemm(L.RQ_MXFP4, a, s, w, ws, 128, L.RQ_OUT_F32)
    assert torch.count_nonzero(y).item() == 0
