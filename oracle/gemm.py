"""Block-scaled GEMM: Y = deq(A) . deq(W)^T, K-major operands.

Oracle (test infrastructure).  The contraction is a plain definition: the
ARCQuant page (technical summary, "Methodologie", unified GEMM execution)
maps the whole computation onto one matrix product whose accumulator adds
every K term, and the Day-0 page (section V item 3) applies the block scales
inside the multiply-accumulate rather than through an intermediate tensor.
Both read as: Y[m, n] = sum_b 2**(ea[m,b] + ew[n,b] - 254) *
sum_{k in b} qa[m,k] * qw[n,k], accumulated in high precision, then rounded
once to the output type.

The oracle forms the dequantized operands in float64 and multiplies them
with NumPy's float64 matmul (a library primitive serving as one step).  For
MXFP4 every product has at most 4 significant bits and the partial sums of
the workloads used here stay exact in float64; ``exact_matmul`` (Python
Fractions) is the brute-force pin on tiny shapes.

Output rounding to BF16 goes straight from float64 (one rounding).
"""

from fractions import Fraction

import numpy as np

from . import formats as F
from . import quant as Q


def matmul_f64(a, w):
    """a [M, K] float64, w [N, K] float64 -> a @ w.T in float64."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T


def exact_matmul(a, w):
    """Exact rational a @ w.T for tiny float64 inputs (brute force)."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, K = a.shape
    N = w.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(a[m, k])) * Fraction(float(w[n, k]))
            out[m][n] = s
    return out


def gemm_mx(a_codes, a_scales, w_codes, w_scales, fmt):
    """Block-scaled GEMM on unpacked codes; returns float64 [M, N]."""
    a = Q.dequantize_mx(a_codes, a_scales, fmt)
    w = Q.dequantize_mx(w_codes, w_scales, fmt)
    return matmul_f64(a, w)


def gemm_bf16(a_bits, w_bits):
    """BF16 x BF16 with a high-precision accumulator; float64 [M, N]."""
    return matmul_f64(F.bf16_to_f64(a_bits), F.bf16_to_f64(w_bits))


def abs_bound(a, w):
    """Per-element sum_k |a_k * w_k| (float64), for the per-element
    tolerance max|gpu - oracle| <= 1e-3 * sum_k |a_k w_k|."""
    return matmul_f64(np.abs(a), np.abs(w))


def rel_frobenius(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    return num / den if den > 0 else num


def to_bf16(y):
    """float64 result -> BF16 bits (one rounding)."""
    return F.f64_to_bf16(y)
