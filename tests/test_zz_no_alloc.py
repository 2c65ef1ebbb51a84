"""rq_escalation_gate_noalloc (per-range statistics in the library's static
device scratch) against rq_escalation_gate with a caller workspace: the
same flags and statistics bit for bit, on two calls in a row, the second
with a smaller input, so the second reads none of the first's leftovers."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from tests.gpu_util import dev_bf16, host, log

pytestmark = pytest.mark.gpu


def with_workspace(z, B, V, tau, delta):
    wsb = L.rq_escalation_gate_workspace_bytes(B, V)
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    flags = torch.empty(B, dtype=torch.uint8, device="cuda")
    stats = torch.empty((B, 2), dtype=torch.float32, device="cuda")
    L.rq_escalation_gate(z, B, V, tau, delta, flags, stats, ws, wsb)
    return host(flags), host(stats)


def no_alloc(z, B, V, tau, delta):
    flags = torch.full((B,), 0xEE, dtype=torch.uint8, device="cuda")
    stats = torch.full((B, 2), np.nan, dtype=torch.float32, device="cuda")
    L.rq_escalation_gate_noalloc(z, B, V, tau, delta, flags, stats)
    return host(flags), host(stats)


def test_no_alloc_gate_matches_workspace_gate_twice():
    rng = np.random.default_rng(77)
    for B, V, tau, delta in ((16, 151936, 9.0, 0.05), (5, 50001, 7.0, 0.2)):
        z = dev_bf16(F.f64_to_bf16(rng.standard_normal((B, V)) * rng.uniform(0.5, 8.0, (B, 1))))
        log(f"no-alloc gate B={B} V={V}")
        f0, s0 = with_workspace(z, B, V, tau, delta)
        f1, s1 = no_alloc(z, B, V, tau, delta)
        assert np.array_equal(f1, f0), (f1, f0)
        assert np.array_equal(s1.view(np.uint32), s0.view(np.uint32))
        assert 0 < f0.sum() < B  # the thresholds split the rows


def test_no_alloc_gate_rejects_bad_shapes():
    z = torch.zeros((17, 64), dtype=torch.int16, device="cuda")
    flags = torch.empty(17, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.RQError):
        L.rq_escalation_gate_noalloc(z, 17, 64, 1.0, 0.1, flags, None)
