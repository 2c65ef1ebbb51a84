"""RAMP recurrent-depth prefill: one shared block applied for r steps, with a
per-step precision schedule.

Oracle (test infrastructure).  Follows the RAMP page (RAMP: Recurrent
Adaptive Mixed Precision for Efficient Prefill in Recurrent-Depth Language
Models):

* section 2.1: a shared transformation is applied repeatedly to the hidden
  representation, with the same parameters at every step;
* section 2.2: during prefill the whole sequence is processed at every step;
* section 2.3: a precision schedule assigns a precision to each step;
* section 4.1: low precision before the switch step, reference precision
  after it;
* section 4.2: in a low-precision step the eligible dense linears use
  low-precision weights (quantized once) and dynamically quantized
  activations; hidden representations and all other operations stay BF16.

The shared block of the synthetic workload is the token-wise residual MLP
h <- h + W2 . SiLU(W1 . RMSNorm(h)).  Readings:

* Every op boundary rounds to BF16: n = bf16(RMSNorm(h)),
  z = bf16(n W1^T), u = bf16(SiLU(z)), v = bf16(u W2^T), h = bf16(h + v).
* RMSNorm has eps = 1e-6 and no gain vector; SiLU(z) = z / (1 + e^-z).
* Both linears are "eligible": in a quantized step the activations n and u
  are block-quantized afresh and the weights use their one-time quantized
  copies; the GEMM then acts on the dequantized operands.
* Schedule bit t-1 set means step t (1-based) runs quantized.

Each op is computed in float64 and rounded once.
"""

import numpy as np

from . import formats as F
from . import quant as Q
from . import gemm as G

EPS = 1e-6


def rmsnorm(h, eps=EPS):
    """h [S, D] float64 -> h / sqrt(mean(h^2) + eps), no gain."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def quantize_weights(w_bits, fmt):
    """The one-time weight quantization: float64 deq(Q(W))."""
    return Q.quantize_dequantize(w_bits, fmt)


def ramp_step(h_bits, w1_bits, w2_bits, quantized, fmt=F.FMT_MXFP4,
              w1_deq=None, w2_deq=None, eps=EPS):
    """One application of the shared block; returns the new h (BF16 bits)."""
    h = F.bf16_to_f64(h_bits)
    n_bits = F.f64_to_bf16(rmsnorm(h, eps))
    if quantized:
        if w1_deq is None:
            w1_deq = quantize_weights(w1_bits, fmt)
        if w2_deq is None:
            w2_deq = quantize_weights(w2_bits, fmt)
        a1 = Q.quantize_dequantize(n_bits, fmt)
        w1 = w1_deq
    else:
        a1 = F.bf16_to_f64(n_bits)
        w1 = F.bf16_to_f64(w1_bits)
    z_bits = F.f64_to_bf16(G.matmul_f64(a1, w1))
    u_bits = F.f64_to_bf16(silu(F.bf16_to_f64(z_bits)))
    if quantized:
        a2 = Q.quantize_dequantize(u_bits, fmt)
        w2 = w2_deq
    else:
        a2 = F.bf16_to_f64(u_bits)
        w2 = F.bf16_to_f64(w2_bits)
    v_bits = F.f64_to_bf16(G.matmul_f64(a2, w2))
    return F.f64_to_bf16(h + F.bf16_to_f64(v_bits))


def step_is_quantized(schedule, t):
    """Step t (1-based) is quantized when bit t-1 of the schedule is set."""
    return bool((int(schedule) >> (t - 1)) & 1)


def ramp_prefill(h0_bits, w1_bits, w2_bits, schedule, steps, fmt=F.FMT_MXFP4,
                 eps=EPS, return_trajectory=False):
    """Run `steps` applications of the block under `schedule`."""
    w1_deq = w2_deq = None
    if int(schedule) & ((1 << steps) - 1):
        w1_deq = quantize_weights(w1_bits, fmt)  # weights quantized once
        w2_deq = quantize_weights(w2_bits, fmt)
    h = np.asarray(h0_bits, dtype=np.uint16)
    traj = [h]
    for t in range(1, steps + 1):
        h = ramp_step(h, w1_bits, w2_bits, step_is_quantized(schedule, t), fmt,
                      w1_deq, w2_deq, eps)
        traj.append(h)
    return traj if return_trajectory else h


def schedule_mask(quantized_steps):
    """Bitmask from a list of 1-based quantized step numbers."""
    m = 0
    for t in quantized_steps:
        m |= 1 << (t - 1)
    return m


def ramp_schedule(steps, switch):
    """RAMP: steps 1..switch quantized, switch+1..steps reference precision."""
    return schedule_mask(range(1, switch + 1))


def early_bf16_schedule(steps, n_bf16):
    """The reverse placement: the first n_bf16 steps BF16, the rest quantized."""
    return schedule_mask(range(n_bf16 + 1, steps + 1))


def hidden_relative_error(h_bits, ref_bits):
    """Final hidden-state relative error ||h - ref||_F / ||ref||_F."""
    return G.rel_frobenius(F.bf16_to_f64(h_bits), F.bf16_to_f64(ref_bits))
