"""GPU parity of the nibble planes and rq_gemv_nibble_escalate."""

import numpy as np
import pytest
import torch

from mixed_precision_block_amd import api
from mixed_precision_block_amd import _lib as L
from oracle import formats as F
from oracle import gemv as V
from synthetic import workloads as W
from tests import _golden as gold
from tests.gpu_util import COUNTER_BYTES, check_bf16, dev, dev_bf16, host, host_bits, log

pytestmark = pytest.mark.gpu


def tiled_planes(w, scales):
    """The row-tiled plane layout documented for rq_pack_nibble_planes,
    built on the host from the oracle's nibbles."""
    hi, lo = V.split_nibbles(w)
    h4 = hi.astype(np.uint8) & 0xF
    N, K = w.shape
    Np, nb = (N + 63) // 64 * 64, K // 32

    def plane(nib):
        p = np.zeros((Np, K), np.uint8)
        p[:N] = nib
        blk = p.reshape(Np, nb, 4, 8)  # [row, block, dword q, element 8q + e]
        out = np.zeros((Np, nb, 4), np.uint32)
        for j in range(4):
            out |= blk[..., 2 * j].astype(np.uint32) << (4 * j)
            out |= blk[..., 2 * j + 1].astype(np.uint32) << (16 + 4 * j)
        # chunk order: (row tile, block, row within tile)
        return out.reshape(Np // 64, 64, nb, 4).transpose(0, 2, 1, 3).reshape(-1).view(np.uint8)

    s = np.zeros((Np, nb), np.uint16)
    s[:N] = np.asarray(scales, np.float16).view(np.uint16)
    st = s.reshape(Np // 64, 64, nb).transpose(0, 2, 1).reshape(-1)
    return plane(h4), plane(lo), st


def gpu_planes(w, scales):
    return api.pack_nibble_planes(dev(w), dev(np.asarray(scales, np.float16).view(np.int16)))


def test_pack_layout():
    d = W.c5_linear(0, N=200, K=96)
    hi, lo, st = gpu_planes(d["w"], d["scales"])
    th, tl, ts = tiled_planes(d["w"], d["scales"])
    assert np.array_equal(host(hi), th)
    assert np.array_equal(host(lo), tl)
    assert np.array_equal(host(st).view(np.uint16), ts)


def run(x, w, scales, flags, phase, N, split=True):
    planes = gpu_planes(w, scales)
    fl = None if flags is None else dev(np.asarray(flags, np.uint8))
    return host_bits(api.gemv_nibble_escalate(dev_bf16(x), N, planes, fl, phase, split=split))


def test_worked_example():
    g = gold.keyed("gemv_worked.txt")
    w = np.zeros((2, 32), np.int8)
    w[0, :6] = [127, -128, -1, 16, 15, -17]
    w[1, :] = 16
    s = np.array([[0.5], [0.25]], np.float16)
    x = np.zeros((2, 32))
    x[0, :6] = 1.0
    x[1, 0], x[1, 5] = 2.0, -1.0
    xb = F.f64_to_bf16(x)
    assert F.bf16_to_f64(run(xb, w, s, None, L.RQ_LOW, 2)).ravel().tolist() == g["y_low"]
    assert F.bf16_to_f64(run(xb, w, s, [1, 1], L.RQ_BOTH, 2)).ravel().tolist() == g["y_full"]
    assert F.bf16_to_f64(run(xb, w, s, [0, 1], L.RQ_BOTH, 2)).ravel().tolist() == g["y_mixed"]


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("B", [1, 2, 5, 8, 9, 16])
@pytest.mark.parametrize("N,K", [(200, 96), (64, 32), (1000, 1024), (130, 3072)])
def test_small_against_oracle(B, N, K, split):
    """Few row tiles: with a workspace the launch splits K over workgroups
    (slices of 1..32 blocks, some empty), without one it does not."""
    d = W.c5_linear(3, B=B, N=N, K=K)
    flags = np.zeros(B, np.uint8)
    flags[::3] = 1
    log(f"gemv B={B} N={N} K={K} split={split} workspace={L.rq_gemv_workspace_bytes(B, N, K)}")
    y_low = run(d["x"], d["w"], d["scales"], None, L.RQ_LOW, N, split)
    hi, _ = V.split_nibbles(d["w"])
    check_bf16(y_low, V.low_pass(d["x"], d["w"], d["scales"]),
               V.abs_bound(d["x"], 16 * hi.astype(np.int64), d["scales"]), "low pass", k=K)
    y = run(d["x"], d["w"], d["scales"], flags, L.RQ_BOTH, N, split)
    ref = V.low_pass(d["x"], d["w"], d["scales"])
    ref[flags == 1] = V.full_pass(d["x"][flags == 1], d["w"], d["scales"])
    bound = V.abs_bound(d["x"], d["w"], d["scales"]) + V.abs_bound(d["x"], 16 * hi.astype(np.int64), d["scales"])
    check_bf16(y, ref, bound, "low + escalation", k=K)
    assert np.array_equal(y[flags == 0], y_low[flags == 0])


def test_escalate_without_flags_leaves_output():
    d = W.c5_linear(1, B=4, N=128, K=64)
    planes = gpu_planes(d["w"], d["scales"])
    y = torch.full((4, 128), 12345, dtype=torch.int16, device="cuda")
    api.gemv_nibble_escalate(dev_bf16(d["x"]), 128, planes, dev(np.zeros(4, np.uint8)), L.RQ_ESCALATE, y=y)
    assert torch.all(y == 12345).item()


def test_lm_head_full_size_sampled():
    i = len(W.c5_linear_list()) - 1
    d = W.c5_linear(i)
    N, K = 151936, 1024
    y = run(d["x"], d["w"], d["scales"], d["flags"], L.RQ_BOTH, N)
    cols = np.sort(np.random.default_rng(8).choice(N, 2048, replace=False))
    w_s, s_s = d["w"][cols], d["scales"][cols]
    ref = V.low_pass(d["x"], w_s, s_s)
    fl = d["flags"] == 1
    ref[fl] = V.full_pass(d["x"][fl], w_s, s_s)
    hi, _ = V.split_nibbles(w_s)
    bound = V.abs_bound(d["x"], w_s, s_s) + V.abs_bound(d["x"], 16 * hi.astype(np.int64), s_s)
    n = check_bf16(y[:, cols], ref, bound, "LM head", k=K)
    log(f"LM head: {n} of {ref.size} sampled outputs one BF16 step off")


def test_one_layer_full():
    for i in range(7):
        d = W.c5_linear(i)
        N, K = d["w"].shape
        y = run(d["x"], d["w"], d["scales"], d["flags"], L.RQ_BOTH, N)
        ref = V.low_pass(d["x"], d["w"], d["scales"])
        fl = d["flags"] == 1
        ref[fl] = V.full_pass(d["x"][fl], d["w"], d["scales"])
        hi, _ = V.split_nibbles(d["w"])
        bound = V.abs_bound(d["x"], d["w"], d["scales"]) + V.abs_bound(d["x"], 16 * hi.astype(np.int64), d["scales"])
        check_bf16(y, ref, bound, d["name"], k=K)


def test_deterministic():
    d = W.c5_linear(4)
    a = run(d["x"], d["w"], d["scales"], d["flags"], L.RQ_BOTH, d["w"].shape[0])
    b = run(d["x"], d["w"], d["scales"], d["flags"], L.RQ_BOTH, d["w"].shape[0])
    assert np.array_equal(a, b)


def test_split_workspace_reused_across_calls():
    """One workspace serves consecutive split calls of different shapes and
    phases; every output equals a fresh-workspace run and the oracle.  Only
    its first 32 KiB (the arrival counters) is zeroed, once: stale partial
    sums must not matter, and every call leaves the counters zero."""
    wsb = max(L.rq_gemv_workspace_bytes(16, n, k) for n, k in ((1000, 1024), (130, 3072), (64, 256)))
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda")
    ws[:COUNTER_BYTES].zero_()
    for rep in range(2):
        for i, (n, k) in enumerate(((1000, 1024), (130, 3072), (64, 256))):
            d = W.c5_linear(i + 2, B=16, N=n, K=k)
            planes = gpu_planes(d["w"], d["scales"])
            fl = dev(d["flags"])
            x = dev_bf16(d["x"])
            y = torch.empty((16, n), dtype=torch.int16, device="cuda")
            hi, lo, st = planes
            assert L.rq_gemv_workspace_bytes(16, n, k) > 0
            L.rq_gemv_nibble_escalate(x, 16, k, n, hi, lo, st, fl, L.RQ_BOTH, ws, wsb, None, y)
            fresh = host_bits(api.gemv_nibble_escalate(x, n, planes, fl, L.RQ_BOTH))
            assert np.array_equal(host_bits(y), fresh), (rep, n, k)
            ref = V.low_pass(d["x"], d["w"], d["scales"])
            f = d["flags"] == 1
            ref[f] = V.full_pass(d["x"][f], d["w"], d["scales"])
            hi8, _ = V.split_nibbles(d["w"])
            bound = V.abs_bound(d["x"], d["w"], d["scales"]) + V.abs_bound(d["x"], 16 * hi8.astype(np.int64),
                                                                            d["scales"])
            check_bf16(host_bits(y), ref, bound, f"reuse {n}x{k}", k=k)
            assert torch.count_nonzero(ws[:COUNTER_BYTES]).item() == 0, "arrival counters not reset"


@pytest.mark.parametrize("B", [1, 5, 16])
def test_grouped_equals_per_problem(B):
    """One grouped launch over mixed shapes (ragged N, one problem without a
    low plane) gives the per-problem unsplit outputs bit for bit, in both
    phases; a tile total beyond the plan changes nothing."""
    shapes = [(200, 96), (64, 32), (1000, 1024), (130, 3072), (777, 256), (64, 64)]
    rng = np.random.default_rng(B)
    f = rng.random(B) < 0.5
    f[0] = True
    flags = dev(f.astype(np.uint8))
    probs, want_low, want_both = [], [], []
    for i, (n, k) in enumerate(shapes):
        d = W.c5_linear(10 + i, N=n, K=k, B=B)
        planes = gpu_planes(d["w"], d["scales"])
        x = dev_bf16(d["x"])
        if i == 4:
            planes = (planes[0], None, planes[2])
        want_low.append(host_bits(api.gemv_nibble_escalate(x, n, planes, None, L.RQ_LOW, split=False)))
        want_both.append(host_bits(api.gemv_nibble_escalate(x, n, planes, flags, L.RQ_BOTH, split=False))
                         if planes[1] is not None else want_low[-1])
        probs.append((x, planes, torch.zeros((B, n), dtype=torch.bfloat16, device="cuda")))
    table = api.gemv_group(probs)
    assert table[2] == sum((n + 63) // 64 for n, _ in shapes)
    for phase, want in ((L.RQ_LOW, want_low), (L.RQ_BOTH, want_both)):
        for _, _, y in probs:
            y.zero_()
        api.gemv_nibble_escalate_grouped(table, B, flags if phase == L.RQ_BOTH else None, phase)
        for i, (w, (_, _, y)) in enumerate(zip(want, probs)):
            assert np.array_equal(host_bits(y), w), (phase, shapes[i])
    over = (table[0], table[1], table[2] + 5)
    api.gemv_nibble_escalate_grouped(over, B, flags, L.RQ_BOTH)
    for i, (w, (_, _, y)) in enumerate(zip(want_both, probs)):
        assert np.array_equal(host_bits(y), w), shapes[i]
    log(f"grouped GEMV B={B}: {len(shapes)} problems, {table[2]} tiles, equal to per-problem calls")


def esc_ref(d, flags):
    ref = V.low_pass(d["x"], d["w"], d["scales"])
    f = np.asarray(flags) == 1
    ref[f] = V.full_pass(d["x"][f], d["w"], d["scales"])
    hi, _ = V.split_nibbles(d["w"])
    bound = V.abs_bound(d["x"], d["w"], d["scales"]) + V.abs_bound(d["x"], 16 * hi.astype(np.int64), d["scales"])
    return ref, bound


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("B", [1, 2, 5, 16])
@pytest.mark.parametrize("N,K", [(200, 96), (1000, 1024), (130, 3072)])
def test_carry_lo_plane_escalation(B, N, K, split):
    """With an FP32 carry the low pass is unchanged (its BF16 output is the
    carry rounded), and an escalation from the carry reads only the lo
    plane (w_hi NULL) yet matches the oracle's 8-bit recompute."""
    d = W.c5_linear(5, B=B, N=N, K=K)
    flags = np.zeros(B, np.uint8)
    flags[1::2] = 1
    flags[-1] = 1  # at least one flagged token, also for B = 1
    planes = gpu_planes(d["w"], d["scales"])
    x, fl = dev_bf16(d["x"]), dev(flags)
    carry = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")  # every row gets written
    y = api.gemv_nibble_escalate(x, N, planes, None, L.RQ_LOW, split=split, carry=carry)
    y_low = host_bits(y)
    assert np.array_equal(y_low, host_bits(api.gemv_nibble_escalate(x, N, planes, None, L.RQ_LOW, split=split)))
    c = host(carry)
    assert np.array_equal(F.f64_to_bf16(c.astype(np.float64)), y_low)  # the BF16 output is the carry rounded
    hi8, _ = V.split_nibbles(d["w"])
    low_ref = V.low_pass(d["x"], d["w"], d["scales"])
    low_bound = V.abs_bound(d["x"], 16 * hi8.astype(np.int64), d["scales"])
    assert np.all(np.abs(c - low_ref) <= 1e-3 * low_bound + 1e-30)
    api.gemv_nibble_escalate(x, N, (None, planes[1], planes[2]), fl, L.RQ_ESCALATE, y=y, split=split, carry=carry)
    got = host_bits(y)
    ref, bound = esc_ref(d, flags)
    n = check_bf16(got, ref, bound, f"carry escalation B={B} {N}x{K} split={split}", k=K)
    assert np.array_equal(got[flags == 0], y_low[flags == 0])
    assert np.array_equal(host(carry), c)  # the carry is read, not written, by the escalation
    log(f"carry escalation B={B} {N}x{K} split={split}: {n} outputs one BF16 step from the oracle")


def test_carry_both_phases_lm_head_sampled():
    """RQ_BOTH with a carry on the LM head (one wave per row tile)."""
    i = len(W.c5_linear_list()) - 1
    d = W.c5_linear(i)
    N, K = 151936, 1024
    planes = gpu_planes(d["w"], d["scales"])
    carry = torch.empty((16, N), dtype=torch.float32, device="cuda")
    y = host_bits(api.gemv_nibble_escalate(dev_bf16(d["x"]), N, planes, dev(d["flags"]), L.RQ_BOTH, carry=carry))
    cols = np.sort(np.random.default_rng(9).choice(N, 2048, replace=False))
    ds = dict(x=d["x"], w=d["w"][cols], scales=d["scales"][cols])
    ref, bound = esc_ref(ds, d["flags"])
    n = check_bf16(y[:, cols], ref, bound, "LM head with carry", k=K)
    log(f"LM head with carry: {n} of {ref.size} sampled outputs one BF16 step off")


def test_grouped_with_carry_equals_per_problem():
    """Grouped launches where some problems carry FP32 sums: each problem's
    outputs equal its own unsplit call with the same carry choice."""
    B = 16
    shapes = [(200, 96), (1000, 1024), (130, 3072), (64, 64)]
    flags = dev(W.c5_flags(B))
    probs, want = [], []
    for i, (n, k) in enumerate(shapes):
        d = W.c5_linear(20 + i, N=n, K=k, B=B)
        planes = gpu_planes(d["w"], d["scales"])
        x = dev_bf16(d["x"])
        use = i % 2 == 0
        c1 = torch.empty((B, n), dtype=torch.float32, device="cuda") if use else None
        want.append(host_bits(api.gemv_nibble_escalate(x, n, planes, flags, L.RQ_BOTH, split=False, carry=c1)))
        c2 = torch.empty((B, n), dtype=torch.float32, device="cuda") if use else None
        probs.append((x, planes, torch.zeros((B, n), dtype=torch.bfloat16, device="cuda"), c2))
    table = api.gemv_group(probs)
    api.gemv_nibble_escalate_grouped(table, B, flags, L.RQ_BOTH)
    for i, (w, p) in enumerate(zip(want, probs)):
        assert np.array_equal(host_bits(p[2]), w), shapes[i]
