"""Helpers for the GPU parity tests: host<->device moves of bit patterns and
the tolerance checks (per element |gpu - oracle| <= 1e-3 * sum_k |a_k w_k|,
relative Frobenius <= 1e-5 on FP32 outputs, BF16 outputs within one BF16
unit in the last place of the oracle's correctly rounded value)."""

import sys

import numpy as np
import torch

from oracle import formats as F

DEV = "cuda"
REL_FRO = 1e-5
PER_ELEM = 1e-3
# the split-K GEMV workspace starts with its arrival counters, one per
# 128-byte line for up to 256 row tiles (include/rq.h, rq_gemv_nibble_escalate)
COUNTER_BYTES = 32768


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    """uint16 BF16 bit patterns -> int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bits(t):
    """Device BF16 (any 2-byte dtype) -> uint16 numpy."""
    torch.cuda.synchronize()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm(ref)
    return np.linalg.norm(y - ref) / (d if d > 0 else 1.0)


def check_f32(y, ref, bound, what="", rel=REL_FRO):
    """FP32 result against the float64 oracle: relative Frobenius and the
    per-element bound."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - ref)
    worst = np.max(err - PER_ELEM * bound) if err.size else -1
    rf = rel_fro(y, ref)
    assert rf <= rel, f"{what}: relative Frobenius {rf:.3e} > {rel}"
    assert worst <= 0, f"{what}: per-element bound exceeded by {worst:.3e}"
    return rf


def bf16_ulp_dist(a_bits, b_bits):
    """Distance in BF16 steps between two arrays of BF16 bit patterns
    (ordered as signed magnitudes, so -0 and +0 are 0 apart)."""
    def key(b):
        b = np.asarray(b, np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(key(a_bits) - key(b_bits))


def check_bf16(y_bits, ref_f64, bound, what="", max_ulp=1, k=None):
    """BF16 result: within max_ulp of the correctly rounded oracle value,
    except where the FP32 accumulation itself may move it further -- outputs
    that cancel to far below sum_k |a_k w_k| -- where the error must stay
    within the FP32 accumulation bound (k + 16) 2^-24 sum_k |a_k w_k|
    (k = reduction length).
    Everything stays inside the per-element bound."""
    ref_bits = F.f64_to_bf16(ref_f64)
    d = bf16_ulp_dist(y_bits, ref_bits)
    err = np.abs(F.bf16_to_f64(y_bits) - ref_f64)
    acc_bound = np.inf if k is None else (k + 16) * 2.0 ** -24 * np.asarray(bound)
    bad = (d > max_ulp) & ~(err <= acc_bound + np.abs(ref_f64) * 2.0 ** -8)
    assert not bad.any(), f"{what}: {int(d[bad].max())} BF16 ulps off at {np.argwhere(bad)[:3].tolist()}"
    # the output rounding adds half a BF16 step of the value to the bound
    slack = np.abs(ref_f64) * 2.0 ** -8
    assert np.all(err <= PER_ELEM * bound + slack), f"{what}: per-element bound exceeded"
    return int((d > 0).sum())
