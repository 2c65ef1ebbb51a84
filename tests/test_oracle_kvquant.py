"""Pins for oracle/kvquant.py: torch running the Day-0 listing itself on
float32 tiles of 128, plus the all-zero tile special case."""

import numpy as np
import torch

from oracle import formats as F
from oracle import kvquant as KV
from synthetic import workloads as W


def test_matches_listing_run_in_torch():
    x = W.kv_tiles(T=64, H=4, D=256)["x"]
    codes, scales = KV.quantize_kv(x)
    t = torch.from_numpy(F.bf16_to_f64(x).astype(np.float32)).reshape(-1, 128)
    amax = t.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    assert np.array_equal(codes.reshape(-1, 128), q.view(torch.uint8).numpy())
    assert np.array_equal(scales.reshape(-1), scale.reshape(-1).numpy())


def test_zero_tile():
    x = np.zeros((1, 1, 256), np.uint16)
    x[0, 0, 200] = F.f64_to_bf16(np.array([3.5]))[0]
    codes, scales = KV.quantize_kv(x)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, :128] == 0)
    assert scales[0, 0, 1] == np.float32(3.5) / np.float32(448.0)
    assert codes[0, 0, 200] == 0x7E  # the tile max maps to 448


def test_roundtrip_error_bound():
    x = W.kv_tiles(T=32, H=2, D=128)["x"]
    codes, scales = KV.quantize_kv(x)
    xv = F.bf16_to_f64(x)
    err = np.abs(KV.dequantize_kv(codes, scales) - xv)
    amax = np.abs(xv).reshape(32, 2, 1, 128).max(-1, keepdims=True)
    # E4M3 relative step is 2**-3 of the element's binade, 2**-9 absolute
    # below the normal range: half a step bounds the error
    bound = np.maximum(np.abs(xv) * 2.0 ** -4, (amax / 448.0 * 2.0 ** -10).reshape(32, 2, 1, 1).repeat(128, -1).reshape(32, 2, 128))
    assert np.all(err <= bound * (1 + 1e-6))
