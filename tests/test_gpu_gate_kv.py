"""GPU parity of the escalation gate and the FP8 KV tile quantizer."""

import numpy as np
import pytest

from mixed_precision_block_amd import api
from oracle import formats as F
from oracle import gate as GT
from oracle import kvquant as KV
from synthetic import workloads as W
from tests.gpu_util import dev_bf16, host, log

pytestmark = pytest.mark.gpu


def logits_batch(V=151936):
    rng = np.random.default_rng(9)
    z = rng.standard_normal((8, V)) * np.array([0.5, 1, 2, 3, 4, 6, 8, 12])[:, None]
    z[5, 17] += 40.0  # one confident token
    z[6, 3] = z[6, 9] = z[6].max() + 5.0  # an exact top-2 tie
    return F.f64_to_bf16(z)


@pytest.mark.parametrize("split", [True, False])
def test_gate_stats_and_flags(split):
    z = logits_batch()
    h_o, gap_o = GT.softmax_stats(z)
    for tau, delta in ((5.0, 0.05), (11.0, 0.5), (0.0, 0.0)):
        flags, stats = api.escalation_gate(dev_bf16(z), tau, delta, split=split)
        st = host(stats)
        assert np.allclose(st[:, 0], h_o, rtol=1e-4, atol=1e-4), (st[:, 0], h_o)
        assert np.allclose(st[:, 1], gap_o, rtol=1e-4, atol=1e-6), (st[:, 1], gap_o)
        want = GT.escalation_flags(z, tau, delta)
        clear = (np.abs(h_o - tau) > 1e-3) & (np.abs(gap_o - delta) > 1e-4)
        assert np.array_equal(host(flags)[clear], want[clear])
        log(f"gate split={split} tau={tau} delta={delta}: flags {host(flags).tolist()}")


@pytest.mark.parametrize("B,V", [(16, 151936), (3, 1001), (5, 7), (2, 2), (16, 4097)])
def test_gate_ragged_rows_split_and_whole(B, V):
    """Row lengths that leave rows off 16-byte boundaries (scalar head and
    tail elements), rows shorter than one vector, and a row that splits into
    ranges with a short last one: both launch forms against the oracle."""
    rng = np.random.default_rng(B * 100003 + V)
    z = F.f64_to_bf16(rng.standard_normal((B, V)) * rng.uniform(0.5, 6.0, (B, 1)))
    h_o, gap_o = GT.softmax_stats(z)
    got = {}
    for split in (True, False):
        flags, stats = api.escalation_gate(dev_bf16(z), 1.0, 0.01, split=split)
        st = host(stats)
        assert np.allclose(st[:, 0], h_o, rtol=1e-4, atol=1e-4), (split, st[:, 0], h_o)
        assert np.allclose(st[:, 1], gap_o, rtol=1e-4, atol=1e-6), (split, st[:, 1], gap_o)
        got[split] = st
    assert np.allclose(got[True], got[False], rtol=1e-5, atol=1e-6)
    log(f"gate B={B} V={V}: split and whole-row statistics agree with the oracle")


@pytest.mark.parametrize("T,H,D", [(256, 8, 128), (37, 3, 256), (1, 1, 128)])
def test_kv_quant_bit_exact(T, H, D):
    x = W.kv_tiles(T=T, H=H, D=D)["x"]
    codes, scales = api.kv_quantize(dev_bf16(x))
    oc, os_ = KV.quantize_kv(x)
    assert np.array_equal(host(scales), os_)
    assert np.array_equal(host(codes), oc)


def test_kv_quant_rounding_boundaries():
    """Tiles whose amax is 448 have scale 1, so x / scale is x itself: BF16
    values placed on every E4M3 rounding tie (normal binades and the
    subnormal range), both signs, -0 and BF16 subnormals pin the encoding of
    the clipped quotients to the oracle's round-to-nearest-even bit for bit."""
    mids = [(1 + (2 * j + 1) / 16) * 2.0 ** e for e in range(-6, 9) for j in range(8)]
    mids = [m for m in mids if m < 448]                      # ties between normal codes
    subs = [(2 * m + 1) * 2.0 ** -10 for m in range(8)]     # ties in the subnormal range
    exact = [k * 2.0 ** -9 for k in range(16)] + [2.0 ** e for e in range(-9, 9)]
    tiny = [2.0 ** -133, 2.0 ** -127, 2.0 ** -126, 2.0 ** -11]  # BF16 subnormals and quotients far below 2^-9
    vals = mids + subs + exact + tiny
    vals = vals + [-v for v in vals] + [-0.0]
    tiles = []
    for i in range(0, len(vals), 127):
        chunk = vals[i:i + 127]
        tiles.append([448.0] + chunk + [0.0] * (127 - len(chunk)))
    x = np.asarray(tiles, np.float64).reshape(len(tiles), 1, 128)
    bits = F.f64_to_bf16(x)
    assert np.array_equal(F.bf16_to_f64(bits), x), "every probe value is a BF16 value"
    codes, scales = api.kv_quantize(dev_bf16(bits))
    oc, os_ = KV.quantize_kv(bits)
    assert np.array_equal(host(scales), os_)
    assert np.all(host(scales) == 1.0)
    assert np.array_equal(host(codes), oc)
    log(f"KV rounding boundaries: {len(vals)} values in {len(tiles)} tiles encode as the oracle does")
