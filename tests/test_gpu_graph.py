"""HIP-graph capture of library calls: a captured sequence (quantize + GEMM,
nibble GEMVs including the split-K partial sums and their reduction, two of
them through the FP32 carry, a short recurrent prefill whose quantized
steps quantize u in the GEMM epilogue, and the escalation gate split over
ranges with its merge) replays to the eager results, bit for
bit, on every replay, with eager work and synchronizations between the
replays.  Nothing the library launches records a memset, so the captured
graph holds only kernel nodes."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from synthetic import workloads as W
from tests.gpu_util import dev, dev_bf16, log

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch.cuda.synchronize()
    # quantize + GEMM of one layer group (4096 x 1024 input, 4096 x 1024 weights)
    g = W.c2_layer(M=1024)[0]
    a = dev_bf16(g["a"])
    wq = api.quantize(dev_bf16(g["w"]), L.RQ_MXFP8)
    M, K = g["a"].shape
    N = g["w"].shape[0]
    ac = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    # three GEMVs: one split over K (workspace), one unsplit, and the escalation of flagged tokens
    gemvs = []
    for i, (n, k) in enumerate(((1024, 1024), (20000, 1024), (1024, 3072))):
        d = W.c5_linear(i, N=n, K=k)
        planes = api.pack_nibble_planes(dev(d["w"]), dev(np.asarray(d["scales"], np.float16).view(np.int16)))
        wsb = L.rq_gemv_workspace_bytes(16, n, k)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")  # arrival counters start at zero
        carry = torch.empty((16, n), dtype=torch.float32, device="cuda") if i < 2 else None
        gemvs.append(dict(x=dev_bf16(d["x"]), planes=planes, n=n, k=k, ws=ws, wsb=wsb, carry=carry,
                          flags=dev(d["flags"]), y=torch.empty((16, n), dtype=torch.int16, device="cuda")))
    # a short recurrent prefill: steps 1-2 MXFP4 (u quantized in the W1 epilogue), step 3 BF16
    r = W.c4_ramp(S=256, D=256, F=512)
    w1, w2 = dev_bf16(r["w1"]), dev_bf16(r["w2"])
    w1q, w2q = api.quantize(w1, L.RQ_MXFP4), api.quantize(w2, L.RQ_MXFP4)
    h0 = dev_bf16(r["h0"])
    h = h0.clone()
    rws = torch.empty(L.rq_recurrent_prefill_workspace_bytes(256, 256, 512, L.RQ_MXFP4), dtype=torch.uint8,
                      device="cuda")
    # the escalation gate over the second GEMV's outputs (16 x 20000 logits), split over ranges
    gv = gemvs[1]
    gwsb = L.rq_escalation_gate_workspace_bytes(16, gv["n"])
    gws = torch.empty(gwsb, dtype=torch.uint8, device="cuda")
    gflags = torch.empty(16, dtype=torch.uint8, device="cuda")
    gstats = torch.empty((16, 2), dtype=torch.float32, device="cuda")

    def work():
        L.rq_quantize(a, M, K, L.RQ_MXFP8, None, 0, L.RQ_APPEND_NONE, ac, as_)
        L.rq_gemm(L.RQ_MXFP8, ac, as_, wq[0], wq[1], M, N, K, L.RQ_OUT_BF16, y)
        for v in gemvs:
            hi, lo, st = v["planes"]
            L.rq_gemv_nibble_escalate(v["x"], 16, v["k"], v["n"], hi, lo, st, v["flags"], L.RQ_BOTH, v["ws"],
                                      v["wsb"], v["carry"], v["y"])
        L.rq_recurrent_prefill(h, 256, 256, 512, w1, w2, w1q[0], w1q[1], w2q[0], w2q[1], L.RQ_MXFP4, 0b011, 3,
                               1e-6, rws, rws.numel())
        L.rq_escalation_gate(gv["y"], 16, gv["n"], 1.0, 0.01, gflags, gstats, gws, gwsb)

    outs = [ac, as_, y, h, gflags, gstats] + [v["y"] for v in gemvs] + [v["carry"] for v in gemvs
                                                                        if v["carry"] is not None]

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().numpy().copy() for t in outs]

    def clear():
        for t in outs:
            t.zero_()
        h.copy_(h0)  # the prefill runs in place from h0
        torch.cuda.synchronize()

    clear()
    work()
    eager = snapshot()
    assert any(g["wsb"] > 0 for g in gemvs), "the split-K path is part of the capture"
    assert gwsb > 0, "the split gate is part of the capture"
    work()  # warm the capture path on the side stream torch uses for capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        clear()
        graph.replay()
        got = snapshot()
        for i, (e, o) in enumerate(zip(eager, got)):
            assert np.array_equal(e, o), f"replay {rep}: output {i} differs from the eager run"
        # eager work between replays
        clear()
        work()
        again = snapshot()
        for e, o in zip(eager, again):
            assert np.array_equal(e, o)
        log(f"graph replay {rep}: all {len(got)} outputs equal the eager run")
