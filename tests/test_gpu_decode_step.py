"""A decode step in layer order (Escalation page, setup paragraph: the cost
is the weight bytes read per generated token over a real decode, where each
layer's input comes from the layer before).  Two layers of the Qwen3-0.6B
shapes run as q/k/v (stacked, shared input), o, gate/up (stacked), down,
each GEMV's input a slice of the previous GEMV's output on the device, one
stream, one split-K workspace shared by every launch.  Every stage matches
the oracle's low pass with the flagged tokens recomputed at 8 bits, on the
input the GPU actually fed it; a captured HIP graph of the whole step
replays to the eager bits."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import gemv as V
from synthetic import workloads as W
from tests.gpu_util import COUNTER_BYTES, check_bf16, dev, dev_bf16, host_bits, log

pytestmark = pytest.mark.gpu

B = 16
LAYER = (("qkv", 1024, 2048 + 1024 + 1024), ("o", 2048, 1024), ("gate_up", 1024, 2 * 3072), ("down", 3072, 1024))
LAYERS = 2


def build():
    stages = []
    for layer in range(LAYERS):
        for j, (name, K, N) in enumerate(LAYER):
            d = W.c5_linear(4 * layer + j, B=B, N=N, K=K)
            planes = api.pack_nibble_planes(dev(d["w"]), dev(np.asarray(d["scales"], np.float16).view(np.int16)))
            stages.append(dict(name=f"layers.{layer}.{name}", K=K, N=N, w=d["w"], scales=d["scales"],
                               planes=planes, x0=d["x"]))
    return stages


def expected(x_bits, st, flags):
    ref = V.low_pass(x_bits, st["w"], st["scales"])
    f = flags.astype(bool)
    ref[f] = V.full_pass(x_bits[f], st["w"], st["scales"])
    hi, _ = V.split_nibbles(st["w"])
    bound = (V.abs_bound(x_bits, st["w"], st["scales"])
             + V.abs_bound(x_bits, 16 * hi.astype(np.int64), st["scales"]))
    return ref, bound


def test_decode_step_layer_ordered():
    stages = build()
    flags_h = W.c5_flags(B)
    flags = dev(flags_h)
    wsb = max(L.rq_gemv_workspace_bytes(B, s["N"], s["K"]) for s in stages)
    assert wsb > 0, "the step's small-N shapes split K"
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")  # arrival counters start at zero
    xs = [torch.empty((B, s["K"]), dtype=torch.bfloat16, device="cuda") for s in stages]
    ys = [torch.empty((B, s["N"]), dtype=torch.bfloat16, device="cuda") for s in stages]
    x_first = dev_bf16(stages[0]["x0"])

    def step():
        xs[0].copy_(x_first)
        for i, s in enumerate(stages):
            hi, lo, st = s["planes"]
            L.rq_gemv_nibble_escalate(xs[i], B, s["K"], s["N"], hi, lo, st, flags, L.RQ_BOTH, ws, wsb, None, ys[i])
            if i + 1 < len(stages):
                xs[i + 1].copy_(ys[i][:, :stages[i + 1]["K"]])  # the next layer's input, on the device

    def snapshot():
        torch.cuda.synchronize()
        return [host_bits(t) for t in xs] + [host_bits(t) for t in ys]

    step()
    eager = snapshot()
    off = 0
    for i, s in enumerate(stages):
        x_bits, y_bits = eager[i], eager[len(stages) + i]
        ref, bound = expected(x_bits, s, flags_h)
        off += check_bf16(y_bits, ref, bound, f"decode step {s['name']} {s['N']}x{s['K']}", k=s["K"])
    assert torch.count_nonzero(ws[:COUNTER_BYTES]).item() == 0, "arrival counters not reset"

    # the whole step as one captured graph, replayed with eager work between
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for t in xs + ys:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, b in zip(eager, got):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager step"
        step()
        again = snapshot()
        for a, b in zip(eager, again):
            assert np.array_equal(a, b)
    log(f"decode step: {len(stages)} GEMVs in layer order, {off} outputs one BF16 step from the oracle; "
        f"graph replays equal the eager step")
