"""GPU parity of rq_recurrent_prefill: the hand-worked steps, small
schedules against the oracle trajectory, single steps from the oracle's
state, and the full 4096-token workload on sampled rows (the block acts
on each token independently, so a subset of rows is an exact sub-problem)."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from oracle import quant as Q
from oracle import ramp as R
from synthetic import workloads as W
from tests import _golden as gold
from tests import f8mfma_model as FM
from tests.gpu_util import dev_bf16, host_bits, log, rel_fro

pytestmark = pytest.mark.gpu

FMT = {F.FMT_MXFP4: L.RQ_MXFP4, F.FMT_MXFP8: L.RQ_MXFP8}


def gpu_prefill(h0, w1, w2, schedule, steps, ofmt, eps=1e-6, gemm_fmt=None):
    """gemm_fmt: the prefill's fmt when it differs from the code format
    (RQ_MXFP8_F8MFMA: MXFP8 codes, GEMMs on the FP8 scaled instruction)."""
    fmt = FMT[ofmt]
    w1d, w2d = dev_bf16(w1), dev_bf16(w2)
    w1q = api.quantize(w1d, fmt)
    w2q = api.quantize(w2d, fmt)
    h = dev_bf16(h0)
    api.recurrent_prefill(h, w1d, w2d, w1q, w2q, fmt if gemm_fmt is None else gemm_fmt, schedule, steps, eps)
    return host_bits(h)


def test_worked_steps():
    w1 = np.zeros((32, 32))
    w1[:, 0] = 2.0
    w2 = np.zeros((32, 32))
    w2[:, 0] = 1.0
    h0 = np.empty((2, 32))
    h0[0], h0[1] = 3.0, -3.0
    cases = {"bf16_step": (0, 1, F.FMT_MXFP4), "mxfp4_step": (1, 1, F.FMT_MXFP4),
             "mxfp8_step": (1, 1, F.FMT_MXFP8), "bf16_three_steps": (0, 3, F.FMT_MXFP4),
             "sched001_three": (1, 3, F.FMT_MXFP4)}
    for row in gold.rows("ramp_worked_step.txt"):
        case, r, h_want = row[0], int(row[1]), float(row[3])
        if case == "zround_step":
            w1z = np.zeros((32, 32))
            w1z[:, 0], w1z[:, 1] = 1.0, 2.0 ** -9
            h = gpu_prefill(F.f64_to_bf16(np.full((1, 32), 0.25)), F.f64_to_bf16(w1z), F.f64_to_bf16(w2), 0, 1,
                            F.FMT_MXFP4)
        else:
            sched, steps, ofmt = cases[case]
            h = gpu_prefill(F.f64_to_bf16(h0), F.f64_to_bf16(w1), F.f64_to_bf16(w2), sched, steps, ofmt)
        assert F.bf16_to_f64(h)[r].tolist() == [h_want] * 32, case


SCHEDULES = {"all_bf16": 0x00, "ramp_1_6": 0x3F, "uniform": 0xFF, "early_bf16": 0xFC}


def ramp_prefill_f8_instruction(h0, w1, w2, schedule, steps):
    """The oracle's recurrence (its RMSNorm, SiLU, BF16 rounding and MXFP8
    block quantization) with each quantized step's two GEMMs taken by the
    model of the FP8 scaled instruction instead of the exact block-scaled
    sum: the reference for rq_recurrent_prefill(RQ_MXFP8_F8MFMA).  A step's
    truncated products change a few BF16 roundings and MXFP8 codes, and the
    recurrence carries those changes on, so the trajectory is compared with
    this model's rather than with the exact one's."""
    w1c, w1s = Q.quantize_mx(w1, F.FMT_MXFP8)
    w2c, w2s = Q.quantize_mx(w2, F.FMT_MXFP8)
    h = np.asarray(h0, dtype=np.uint16)
    for t in range(1, steps + 1):
        if not R.step_is_quantized(schedule, t):
            h = R.ramp_step(h, w1, w2, False)
            continue
        n_bits = F.f64_to_bf16(R.rmsnorm(F.bf16_to_f64(h)))
        nc, ns = Q.quantize_mx(n_bits, F.FMT_MXFP8)
        z_bits = F.f64_to_bf16(FM.gemm_f8mfma(nc, ns, w1c, w1s))
        u_bits = F.f64_to_bf16(R.silu(F.bf16_to_f64(z_bits)))
        uc, us = Q.quantize_mx(u_bits, F.FMT_MXFP8)
        v_bits = F.f64_to_bf16(FM.gemm_f8mfma(uc, us, w2c, w2s))
        h = F.f64_to_bf16(F.bf16_to_f64(h) + F.bf16_to_f64(v_bits))
    return h


@pytest.mark.parametrize("ofmt,gemm_fmt", [(F.FMT_MXFP4, None), (F.FMT_MXFP8, None),
                                           (F.FMT_MXFP8, L.RQ_MXFP8_F8MFMA)])
def test_small_schedules_against_oracle(ofmt, gemm_fmt):
    """Against the oracle's trajectory at 0.1 x the schedule's own error
    (distance from all-BF16); the FP8 instruction's schedule against the
    oracle's recurrence with the instruction's GEMM model."""
    d = W.c4_ramp(S=96, D=256, F=704)
    ref_bf16 = R.ramp_prefill(d["h0"], d["w1"], d["w2"], 0, 8, ofmt)
    f8 = gemm_fmt == L.RQ_MXFP8_F8MFMA
    for name, sched in SCHEDULES.items():
        if ofmt == F.FMT_MXFP8 and name not in (("ramp_1_6",) if f8 else ("ramp_1_6", "uniform")):
            continue
        g = gpu_prefill(d["h0"], d["w1"], d["w2"], sched, 8, ofmt, gemm_fmt=gemm_fmt)
        if f8:
            o = ramp_prefill_f8_instruction(d["h0"], d["w1"], d["w2"], sched, 8)
        else:
            o = R.ramp_prefill(d["h0"], d["w1"], d["w2"], sched, 8, ofmt)
        err_sched = R.hidden_relative_error(o, ref_bf16)
        err_gpu = rel_fro(F.bf16_to_f64(g), F.bf16_to_f64(o))
        tol = max(1e-3, 0.1 * err_sched)
        log(f"{ofmt} {name}: gpu-vs-oracle {err_gpu:.3e} (tol {tol:.2e}); schedule error vs BF16 {err_sched:.3e}")
        assert err_gpu <= tol


def test_single_steps_from_oracle_state():
    """Each step started from the oracle's h_t: the GPU's h_{t+1} matches in
    nearly every element (rare 1-ulp flips from RMSNorm/exp rounding)."""
    d = W.c4_ramp(S=64, D=256, F=512)
    traj = R.ramp_prefill(d["h0"], d["w1"], d["w2"], 0x0F, 6, F.FMT_MXFP4, return_trajectory=True)
    for t in range(6):
        q = R.step_is_quantized(0x0F, t + 1)
        g = gpu_prefill(traj[t], d["w1"], d["w2"], 1 if q else 0, 1, F.FMT_MXFP4)
        diff = (g != traj[t + 1]).mean()
        err = rel_fro(F.bf16_to_f64(g), F.bf16_to_f64(traj[t + 1]))
        log(f"step {t + 1} ({'MXFP4' if q else 'BF16'}): {diff:.2e} of elements differ, rel {err:.2e}")
        assert err <= 1e-3 and diff <= 0.05


def test_config4_full_size_sampled_rows():
    d = W.c4_ramp()
    rows = np.sort(np.random.default_rng(7).choice(4096, 24, replace=False))
    g = gpu_prefill(d["h0"], d["w1"], d["w2"], 0x3F, 8, F.FMT_MXFP4)[rows]
    o = R.ramp_prefill(d["h0"][rows], d["w1"], d["w2"], 0x3F, 8, F.FMT_MXFP4)
    o_bf = R.ramp_prefill(d["h0"][rows], d["w1"], d["w2"], 0, 8, F.FMT_MXFP4)
    err = rel_fro(F.bf16_to_f64(g), F.bf16_to_f64(o))
    tol = max(1e-3, 0.1 * R.hidden_relative_error(o, o_bf))
    log(f"config-4 RAMP full size, sampled rows: gpu-vs-oracle {err:.3e} (tol {tol:.2e})")
    assert err <= tol


def test_config4_literal_32_step_mxfp8_schedule_sampled_rows():
    """The pages' fixed-budget schedule (RAMP section 4.2: T = 32 steps, the
    first K = 24 in low precision, here MXFP8 W/A, the last 8 BF16) on the
    recurrent block's full shape (4096 tokens, hidden 2048, FFN 5632); the
    oracle runs the sampled rows, which the token-wise block makes an exact
    sub-problem."""
    d = W.c4_ramp()
    sched = (1 << 24) - 1
    rows = np.sort(np.random.default_rng(8).choice(4096, 16, replace=False))
    log("config-4 32-step schedule, steps 1-24 MXFP8")
    g = gpu_prefill(d["h0"], d["w1"], d["w2"], sched, 32, F.FMT_MXFP8)[rows]
    o = R.ramp_prefill(d["h0"][rows], d["w1"], d["w2"], sched, 32, F.FMT_MXFP8)
    o_bf = R.ramp_prefill(d["h0"][rows], d["w1"], d["w2"], 0, 32, F.FMT_MXFP8)
    err = rel_fro(F.bf16_to_f64(g), F.bf16_to_f64(o))
    err_sched = R.hidden_relative_error(o, o_bf)
    tol = max(1e-3, 0.1 * err_sched)
    log(f"gpu-vs-oracle {err:.3e} (tol {tol:.2e}); schedule error vs BF16 {err_sched:.3e}")
    assert err <= tol
