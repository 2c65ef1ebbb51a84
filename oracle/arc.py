"""ARCQuant augmented residual channels on MXFP4.

Oracle (test infrastructure).  Follows the steps of the ARCQuant page
(ARCQuant: Boosting NVFP4 Quantization with Augmented Residual Channels,
technical summary, "Methodologie"), in its order:

1. Outlier identification: rank channels by their absolute maximum over the
   calibration activations and keep the top S.
2. Primary stage: standard block quantization of the activation matrix.
3. Residual stage: for the selected channels, the difference between the
   original value and its primary-quantized value, quantized again into a
   second set of channels of the same 4-bit block format.
4. Augmented product: residual channels are concatenated to the primary
   activations along the reduction dimension K, and the matching weight
   columns are duplicated, so one GEMM over K + S computes primary plus
   correction (the accumulation is linear).

Readings where the page leaves a step open:

* The element format is MXFP4 (E2M1, 32-element blocks, E8M0 scales), the
  page's own extension to MXFP4, not NVFP4's 16-element blocks.
* Selection uses only the amax ranking (top S, S a multiple of 32).  The
  page's extra "significant precision gap" criterion has no threshold, so
  it is not applied.  Ties in amax go to the lower channel index; the order
  of idx is the order of the appended channels.
* No channel reordering of the primary blocks (the page reorders before the
  primary stage; here the primary stage keeps the original order).
* The residual r = x - deq(Q(x)) is formed exactly; it is always a BF16
  value (checked), so keeping it in BF16 loses nothing.
* Appended channels form their own blocks of 32 consecutive j (j indexes
  idx), in the same format as the primary blocks.
* The duplicated weight columns W[:, idx] are quantized in their own new
  blocks (the weights' own K' = K + S block grid).
"""

import numpy as np

from . import formats as F
from . import quant as Q
from . import gemm as G


def select_outlier_channels(x_bits, S):
    """Top-S channels by max_m |x[m, k]|; descending, ties -> lower k."""
    x = F.bf16_to_f64(x_bits)
    c = np.abs(x).max(axis=0)
    order = np.argsort(-c, kind="stable")  # stable: equal c keeps lower k first
    return order[:S].astype(np.int32)


def residual_bits(x_bits, idx, fmt=F.FMT_MXFP4):
    """r[m, j] = x[m, idx[j]] - deq(Q(x))[m, idx[j]] as BF16 bits (exact)."""
    x = F.bf16_to_f64(x_bits)
    deq = Q.quantize_dequantize(x_bits, fmt)
    r = x[:, idx] - deq[:, idx]
    r_bits = F.f64_to_bf16(r)
    if not np.array_equal(F.bf16_to_f64(r_bits), r):
        raise AssertionError("ARC residual is not exactly a BF16 value")
    return r_bits


def augment_activations(x_bits, idx, fmt=F.FMT_MXFP4):
    """A' = [Q(x) | Q(r)]: codes [M, K+S] (unpacked) and scales [M, (K+S)/32]."""
    idx = np.asarray(idx, dtype=np.int64)
    if len(idx) % Q.BLOCK:
        raise ValueError("S must be a multiple of 32")
    pc, ps = Q.quantize_mx(x_bits, fmt)
    if len(idx) == 0:
        return pc, ps
    rc, rs = Q.quantize_mx(residual_bits(x_bits, idx, fmt), fmt)
    return np.concatenate([pc, rc], axis=1), np.concatenate([ps, rs], axis=1)


def augment_weights(w_bits, idx, fmt=F.FMT_MXFP4):
    """W' = Q([W | W[:, idx]]): codes [N, K+S] (unpacked), scales [N, (K+S)/32]."""
    idx = np.asarray(idx, dtype=np.int64)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    w_aug = np.concatenate([w_bits, w_bits[:, idx]], axis=1)
    return Q.quantize_mx(w_aug, fmt)


def copy_append_codes(x_bits, idx, fmt=F.FMT_MXFP4):
    """Codes of Q([x | x[:, idx]]) -- the weight-side append."""
    return augment_weights(x_bits, idx, fmt)


def gemm_arc(a_bits, w_bits, idx, fmt=F.FMT_MXFP4):
    """Y_arc = deq(A') . deq(W')^T in float64."""
    ac, as_ = augment_activations(a_bits, idx, fmt)
    wc, ws = augment_weights(w_bits, idx, fmt)
    return G.gemm_mx(ac, as_, wc, ws, fmt)


def arc_errors(a_bits, w_bits, idx, fmt=F.FMT_MXFP4):
    """Relative Frobenius errors of ARC and plain MX against the float64
    product of the BF16 operands (a reported property: ARC < plain)."""
    ref = G.gemm_bf16(a_bits, w_bits)
    y_arc = gemm_arc(a_bits, w_bits, idx, fmt)
    ac, as_ = Q.quantize_mx(a_bits, fmt)
    wc, ws = Q.quantize_mx(w_bits, fmt)
    y_plain = G.gemm_mx(ac, as_, wc, ws, fmt)
    return G.rel_frobenius(y_arc, ref), G.rel_frobenius(y_plain, ref)
