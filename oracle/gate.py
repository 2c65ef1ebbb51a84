"""Escalation gate over the low-pass logits.

Oracle (test infrastructure).  Follows the escalation article (Escalating
Weight Precision Only When Decoding Becomes Uncertain, setup paragraph):
after the low-precision pass the output distribution is inspected and the
step is recomputed with 8-bit weights when its entropy is above a threshold
or when the gap between the two most likely tokens is small.

Readings: the distribution is softmax over the low-pass logits (one row per
token); entropy is in nats; the gap is p1 - p2 of the two largest
probabilities; a token is flagged when entropy > tau OR gap < delta.  The
thresholds are not printed on the page, so they are parameters.
"""

import numpy as np

from . import formats as F


def softmax_stats(logits_bits):
    """BF16 logits [B, V] -> (entropy [B], p1 - p2 [B]) in float64."""
    z = F.bf16_to_f64(logits_bits)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    entropy = -plogp.sum(axis=1)
    top2 = -np.sort(-p, axis=1)[:, :2]
    return entropy, top2[:, 0] - top2[:, 1]


def escalation_flags(logits_bits, tau, delta):
    """uint8 [B]: 1 where entropy > tau or (p1 - p2) < delta."""
    h, gap = softmax_stats(logits_bits)
    return ((h > tau) | (gap < delta)).astype(np.uint8)
