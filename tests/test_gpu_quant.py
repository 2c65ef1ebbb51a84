"""GPU parity of rq_quantize (codes and scales bit-exact against the
oracle), the ARC append modes, and channel selection (indices bit-exact)."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from oracle import quant as Q
from oracle import arc as A
from synthetic import workloads as W
from tests.gpu_util import dev, dev_bf16, host, log

pytestmark = pytest.mark.gpu

FMTS = [(L.RQ_MXFP4, F.FMT_MXFP4), (L.RQ_MXFP8, F.FMT_MXFP8)]


def finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def gpu_quant(x_bits, fmt, idx=None, append=L.RQ_APPEND_NONE):
    idx_d = None if idx is None else dev(np.asarray(idx, np.int32))
    c, s = api.quantize(dev_bf16(x_bits), fmt, idx_d, append)
    return host(c), host(s)


def assert_same(x_bits, fmt, ofmt, what):
    log(f"quantize {what} fmt={ofmt} shape={x_bits.shape}")
    gc, gs = gpu_quant(x_bits, fmt)
    oc, os_ = Q.quantize_mx(x_bits, ofmt)
    assert np.array_equal(gs, os_), f"{what}: scales differ at {np.argwhere(gs != os_)[:3]}"
    oc = Q.storage_codes(oc, ofmt)
    assert np.array_equal(gc, oc), f"{what}: codes differ at {np.argwhere(gc != oc)[:3]}"


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_exhaustive_value_as_block_max(fmt, ofmt):
    bits = finite_bf16()
    x = np.zeros((bits.size, 32), np.uint16)
    x[:, 0] = bits
    assert_same(x, fmt, ofmt, "every BF16 value as a block max")


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_every_value_under_several_scales(fmt, ofmt):
    """All BF16 magnitudes <= amax, both signs, in blocks whose max is amax."""
    bits = finite_bf16()
    vals = F.bf16_to_f64(bits)
    for amax in (6.0, 448.0, 1.0, 3.0e-38, 1.5e30, 2.0 ** -130):
        sel = bits[np.abs(vals) <= amax]
        n = (sel.size + 30) // 31
        blk = np.zeros((n, 32), np.uint16)
        flat = np.zeros(n * 31, np.uint16)
        flat[:sel.size] = sel
        blk[:, :31] = flat.reshape(n, 31)
        blk[:, 31] = F.f64_to_bf16(np.array([amax]))[0]
        assert_same(blk, fmt, ofmt, f"all values under amax {amax}")


@pytest.mark.parametrize("fmt,ofmt,emax", [(L.RQ_MXFP4, F.FMT_MXFP4, 125), (L.RQ_MXFP8, F.FMT_MXFP8, 119)])
def test_every_value_under_every_block_exponent(fmt, ofmt, emax):
    """For every block exponent e that BF16 inputs can produce, every BF16
    value (both signs) that the scale 2^e covers, in blocks whose max is
    Qmax 2^e (so the block exponent is exactly e)."""
    bits = finite_bf16()
    vals = F.bf16_to_f64(bits)
    qmax = F.FORMATS[ofmt]["qmax"]
    blocks = []
    for e in range(-127, emax + 1):
        amax = qmax * 2.0 ** e
        sel = bits[np.abs(vals) <= amax]
        n = (sel.size + 30) // 31
        flat = np.zeros(n * 31, np.uint16)
        flat[:sel.size] = sel
        blk = np.zeros((n, 32), np.uint16)
        blk[:, :31] = flat.reshape(n, 31)
        blk[:, 31] = F.f64_to_bf16(np.array([amax]))[0]
        blocks.append(blk)
    x = np.concatenate(blocks)
    assert_same(x, fmt, ofmt, f"all values under every block exponent -127..{emax}")


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_workload_tensors(fmt, ofmt):
    assert_same(W.c1_gemm_mxfp4()["a"], fmt, ofmt, "config-1 A")
    assert_same(W.c1_gemm_mxfp4()["w"], fmt, ofmt, "config-1 W")
    assert_same(W.c2_linear(6, M=512)["a"], fmt, ofmt, "config-2 down_proj A (512 rows)")
    assert_same(W.c3_arc()["a"], fmt, ofmt, "config-3 A 4096x4096")
    assert_same(W.c4_ramp(S=512, D=2048, F=64)["h0"], fmt, ofmt, "config-4 h0 (512 rows)")


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (257, 4224), (5, 8192)])
def test_ragged_shapes(fmt, ofmt, rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    x = F.f64_to_bf16(rng.standard_t(3, (rows, K)) * np.exp(rng.uniform(-30, 30, (rows, 1))))
    assert_same(x, fmt, ofmt, "ragged")


def test_adversarial_blocks():
    rng = np.random.default_rng(0)
    rows = []
    for scale in (1.0, 2.0 ** -120, 2.0 ** 100):
        for mids in (F.E2M1_MAGNITUDES, F.E4M3_MAGNITUDES):
            m = 0.5 * (mids[:-1] + mids[1:])  # exact ties of the element grid
            v = np.concatenate([m, -m, [0.0, -0.0]])
            for i in range(0, len(v), 31):
                r = np.zeros(32)
                chunk = v[i:i + 31]
                r[:len(chunk)] = chunk
                r[31] = mids[-1]
                rows.append(r * scale)
    x = F.f64_to_bf16(np.array(rows))
    neg0 = np.signbit(np.array(rows)) & (np.array(rows) == 0)
    x[neg0] = 0x8000
    for fmt, ofmt in FMTS:
        assert_same(x, fmt, ofmt, "ties, zeros, -0, extreme scales")


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("mode", [L.RQ_APPEND_RESIDUAL, L.RQ_APPEND_COPY])
def test_append_modes(fmt, ofmt, mode):
    d = W.c3_arc(M=301, K=512, N=8, n_outliers=16)  # odd: a workgroup with one live row
    rng = np.random.default_rng(mode)
    idx = np.concatenate([A.select_outlier_channels(d["a"], 32), rng.integers(0, 512, 32)]).astype(np.int32)
    idx[40] = idx[3]  # a duplicate channel
    gc, gs = gpu_quant(d["a"], fmt, idx, mode)
    if mode == L.RQ_APPEND_RESIDUAL:
        oc, os_ = A.augment_activations(d["a"], idx, ofmt)
    else:
        oc, os_ = A.copy_append_codes(d["a"], idx, ofmt)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, Q.storage_codes(oc, ofmt))


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("K,S", [(256, 32), (4096, 128), (4096, 2048), (2080, 96), (9600, 2048), (12288, 2080)])
def test_residual_append_extreme_exponents(fmt, ofmt, K, S):
    """Residual appends on blocks whose scale spans BF16's range: rows of
    subnormal BF16 values (block byte 0 or near it), rows near the largest
    finite BF16 and ordinary rows (25 of them: the last workgroup of two
    rows has one live), for the one-pass path (the workgroup's rows in LDS;
    S / 8 appended chunks per row, two rounds of tasks at K = 4096 with
    S = 2048) and, at K = 12288 with S = 2080 (more appended chunks than
    threads), the two-pass path."""
    rng = np.random.default_rng(K + S)
    rows = 25
    mag = rng.standard_normal((rows, K))
    scale = np.concatenate([np.full(8, 2.0 ** -133), np.full(8, 2.0 ** 120), np.ones(9)])
    x = F.f64_to_bf16(mag * scale[:, None])
    idx = rng.integers(0, K, S).astype(np.int32)
    log(f"extreme residual append fmt={ofmt} K={K} S={S}")
    gc, gs = gpu_quant(x, fmt, idx, L.RQ_APPEND_RESIDUAL)
    oc, os_ = A.augment_activations(x, idx, ofmt)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, Q.storage_codes(oc, ofmt))


def test_channel_amax_and_selection():
    for d, S in ((W.c3_arc(), 128), (W.c1_gemm_mxfp4(), 32)):
        x = d["a"]
        amax = api.channel_amax(dev_bf16(x))
        want = np.abs(F.bf16_to_f64(x)).max(axis=0)
        got = F.bf16_to_f64(host(amax).view(np.uint16))
        assert np.array_equal(got, want)
        idx = api.select_channels(amax, S).numpy()
        assert np.array_equal(idx, A.select_outlier_channels(x, S))


def test_deterministic():
    x = W.c3_arc(M=1024, K=1024)["a"]
    a = gpu_quant(x, L.RQ_MXFP4)
    b = gpu_quant(x, L.RQ_MXFP4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_rows_is_a_no_op():
    c = torch.full((4, 16), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((4, 1), 7, dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, 32), dtype=torch.int16, device="cuda")
    L.rq_quantize(x, 0, 32, L.RQ_MXFP4, None, 0, 0, c, s)
    assert int(host(c).min()) == 7 and int(host(s).min()) == 7
