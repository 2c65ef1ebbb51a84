"""Pins for oracle/ramp.py: hand-worked steps, library RMSNorm/SiLU,
invariants of the block and of the schedule helpers."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import ramp as R
from tests import _golden as gold


def worked_weights():
    w1 = np.zeros((32, 32))
    w1[:, 0] = 2.0
    w2 = np.zeros((32, 32))
    w2[:, 0] = 1.0
    return F.f64_to_bf16(w1), F.f64_to_bf16(w2)


def worked_h0():
    h = np.empty((2, 32))
    h[0], h[1] = 3.0, -3.0
    return F.f64_to_bf16(h)


CASES = {
    "bf16_step": (0b0, 1, F.FMT_MXFP4),
    "mxfp4_step": (0b1, 1, F.FMT_MXFP4),
    "mxfp8_step": (0b1, 1, F.FMT_MXFP8),
    "bf16_three_steps": (0b000, 3, F.FMT_MXFP4),
    "sched001_three": (0b001, 3, F.FMT_MXFP4),
    "zround_step": (0b0, 1, F.FMT_MXFP4),
}


@pytest.mark.parametrize("row", gold.rows("ramp_worked_step.txt"), ids=lambda r: f"{r[0]}-{r[1]}")
def test_worked_steps(row):
    case, r, u_want, h_want = row[0], int(row[1]), float(row[2]), float(row[3])
    sched, steps, fmt = CASES[case]
    w1, w2 = worked_weights()
    h0 = worked_h0()
    z = 2.0 if r == 0 else -2.0
    if case == "zround_step":
        w1f = np.zeros((32, 32))
        w1f[:, 0], w1f[:, 1] = 1.0, 2.0 ** -9
        w1 = F.f64_to_bf16(w1f)
        h0 = F.f64_to_bf16(np.full((1, 32), 0.25))
        z = 1.0  # bf16(1 + 2**-9)
    h = R.ramp_prefill(h0, w1, w2, sched, steps, fmt)
    assert F.bf16_to_f64(h)[r].tolist() == [h_want] * 32
    # u after the first step: BF16 SiLU of the BF16 z
    assert F.bf16_to_f64(F.f64_to_bf16(R.silu(np.array([z]))))[0] == u_want


def test_rmsnorm_and_silu_match_torch_float64():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-5, 5, (16, 1)))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (256,), eps=1e-6).numpy()
    assert np.allclose(R.rmsnorm(h, 1e-6), ref, rtol=1e-14, atol=0)
    z = rng.standard_normal(10_000) * 10
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(R.silu(z), ref, rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("sched", [0b0, 0b1])
def test_zero_weights_leave_h_unchanged(sched):
    rng = np.random.default_rng(3)
    h = F.f64_to_bf16(rng.standard_normal((4, 64)))
    w1 = F.f64_to_bf16(rng.standard_normal((96, 64)))
    w2 = F.f64_to_bf16(rng.standard_normal((64, 96)))
    zeros1 = np.zeros_like(w1)
    zeros2 = np.zeros_like(w2)
    assert np.array_equal(R.ramp_prefill(h, w1, zeros2, sched, 1), h)
    assert np.array_equal(R.ramp_prefill(h, zeros1, w2, sched, 1), h)


def test_schedule_helpers():
    assert R.ramp_schedule(8, 6) == 0b00111111
    assert R.early_bf16_schedule(8, 2) == 0b11111100
    assert R.schedule_mask([1, 3]) == 0b101
    assert R.step_is_quantized(0b100, 3) and not R.step_is_quantized(0b100, 2)


def test_quantized_steps_only_where_scheduled():
    """A schedule bit changes only its own step: trajectories agree up to
    the first quantized step and differ from it on."""
    rng = np.random.default_rng(12)
    h = F.f64_to_bf16(rng.standard_normal((8, 64)))
    w1 = F.f64_to_bf16(rng.standard_normal((96, 64)) * 0.1)
    w2 = F.f64_to_bf16(rng.standard_normal((64, 96)) * 0.1)
    ta = R.ramp_prefill(h, w1, w2, 0b000, 3, return_trajectory=True)
    tb = R.ramp_prefill(h, w1, w2, 0b100, 3, return_trajectory=True)
    assert all(np.array_equal(x, y) for x, y in zip(ta[:3], tb[:3]))
    assert not np.array_equal(ta[3], tb[3])
