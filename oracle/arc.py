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
* Two arrangements are built.  augment_activations keeps the original
  channel order for the primary blocks and appends the selected channels'
  residuals (the gather form).  frontend follows the page's fused kernel
  ("Kernel Implementatie": channel reorder, RMSNorm, primary and residual
  quantization in one pass): channels are first permuted by descending
  amax (ties to the lower index), so the S selected channels are the first
  S positions, and the appended residual blocks are those positions'
  residuals.  The "interleaved channel layout ready for the GEMM" is read
  as this reordered [primary | residual] row, the layout the augmented GEMM
  consumes; the weights take the same permutation and the duplicated first
  S columns (frontend with append "copy").
* RMSNorm in the front end is the one of the recurrent block: eps, no gain,
  the normalized value rounded to BF16 before quantization.  The amax
  ranking for the permutation is taken on the normalized activations.
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
from . import ramp as R


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


def reorder_permutation(x_bits):
    """perm[j] = the channel placed at position j: all K channels by
    descending max_m |x[m, k]|, ties -> lower k (so perm[:S] is the top-S
    selection)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    return select_outlier_channels(x_bits, x_bits.shape[1])


def rmsnorm_bits(h_bits, eps=R.EPS):
    """n = bf16(h / sqrt(mean(h^2) + eps)) per row, no gain."""
    return F.f64_to_bf16(R.rmsnorm(F.bf16_to_f64(h_bits), eps))


def frontend(h_bits, perm, S, fmt=F.FMT_MXFP4, append="residual", rmsnorm=True, eps=R.EPS):
    """The fused front end, step by step:
    1. n = rmsnorm_bits(h) (or h itself when rmsnorm is False);
    2. x = n[:, perm] -- the outlier channels move to the first S positions;
    3. primary: block quantization of x over K;
    4. appended S channels: "residual" -> Q(x - deq(Q(x))) of positions
       0..S-1 (activations), "copy" -> Q(x) of positions 0..S-1 (weights).
    Returns codes [rows, K+S] (unpacked) and scales [rows, (K+S)/32]."""
    h_bits = np.asarray(h_bits, dtype=np.uint16)
    perm = np.asarray(perm, dtype=np.int64)
    if sorted(perm.tolist()) != list(range(h_bits.shape[1])):
        raise ValueError("perm must be a permutation of the K channels")
    n = rmsnorm_bits(h_bits, eps) if rmsnorm else h_bits
    x = n[:, perm]
    first = np.arange(S)
    if append == "residual":
        return augment_activations(x, first, fmt)
    if append == "copy":
        return augment_weights(x, first, fmt)
    raise ValueError(append)
