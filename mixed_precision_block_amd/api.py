"""Allocate-and-call wrappers over the rq_* binding.

Outputs are torch tensors on the input's device; BF16 tensors may be given
as torch.bfloat16 or any 2-byte integer view of the bit patterns.  All
arithmetic happens in librq's kernels.
"""

import torch

from . import _lib as L


def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


def code_bytes(fmt, K):
    return K // 2 if fmt == L.RQ_MXFP4 else K


def quantize(x, fmt, idx=None, append=L.RQ_APPEND_NONE, stream=None):
    """x [rows, K] BF16 -> (codes uint8 [rows, K'(/2)], scales uint8 [rows, K'/32])."""
    rows, K = x.shape
    S = 0 if idx is None else int(idx.numel())
    Kp = K + S
    codes = _u8((rows, code_bytes(fmt, Kp)), x.device)
    scales = _u8((rows, Kp // 32), x.device)
    L.rq_quantize(x, rows, K, fmt, idx, S, append, codes, scales, stream)
    return codes, scales


def channel_amax(x, stream=None):
    rows, K = x.shape
    out = torch.empty(K, dtype=torch.int16, device=x.device)
    L.rq_channel_amax(x, rows, K, out, stream)
    return out


def select_channels(amax, S):
    """Top-S channels (host helper); amax on any device, idx returned on CPU."""
    a = amax.detach().to("cpu").contiguous()
    idx = torch.empty(S, dtype=torch.int32)
    L.rq_select_channels(a, a.numel(), S, idx)
    return idx


def arc_frontend(x, perm, S, fmt=L.RQ_MXFP4, append=L.RQ_APPEND_RESIDUAL, rmsnorm=True, eps=1e-6, stream=None):
    """x [rows, K] BF16, perm [K] int32 on the device -> (codes, scales) of the
    reordered, optionally normalized row with S appended channels."""
    rows, K = x.shape
    if S == 0:
        append = L.RQ_APPEND_NONE
    Kp = K + S
    codes = _u8((rows, code_bytes(fmt, Kp)), x.device)
    scales = _u8((rows, Kp // 32), x.device)
    L.rq_arc_frontend(x, rows, K, perm, S, fmt, append, 1 if rmsnorm else 0, eps, codes, scales, stream)
    return codes, scales


def rmsnorm(h, eps=1e-6, stream=None):
    rows, D = h.shape
    out = torch.empty_like(h)
    L.rq_rmsnorm(h, rows, D, eps, out, stream)
    return out


def reorder_permutation(x, stream=None):
    """All channels by descending amax of x (ties to the lower index), as a
    device int32 tensor."""
    K = x.shape[1]
    return select_channels(channel_amax(x, stream), K).to(x.device)


def gemm(fmt, a, a_scales, w, w_scales, K, out=L.RQ_OUT_BF16, stream=None):
    M, N = a.shape[0], w.shape[0]
    dt = torch.float32 if out == L.RQ_OUT_F32 else torch.bfloat16
    y = torch.empty((M, N), dtype=dt, device=a.device)
    L.rq_gemm(fmt, a, a_scales, w, w_scales, M, N, K, out, y, stream)
    return y


def gemm_arc(a, idx, w_aug, w_aug_scales, out=L.RQ_OUT_BF16, workspace=None, stream=None):
    M, K = a.shape
    S = int(idx.numel())
    N = w_aug.shape[0]
    ws_bytes = L.rq_gemm_arc_workspace_bytes(M, K, S)
    if workspace is None:
        workspace = _u8((ws_bytes,), a.device)
    dt = torch.float32 if out == L.RQ_OUT_F32 else torch.bfloat16
    y = torch.empty((M, N), dtype=dt, device=a.device)
    L.rq_gemm_arc(a, M, K, idx, S, w_aug, w_aug_scales, N, workspace, workspace.numel(), out, y, stream)
    return y


def recurrent_prefill(h, w1, w2, w1q, w2q, fmt, schedule, steps, eps=1e-6, workspace=None, stream=None):
    """In place on h [S, D] BF16.  w1q / w2q: (codes, scales) or None."""
    S, D = h.shape
    F = w1.shape[0] if w1 is not None else w1q[0].shape[0]
    ws_bytes = L.rq_recurrent_prefill_workspace_bytes(S, D, F, fmt)
    if workspace is None:
        workspace = _u8((ws_bytes,), h.device)
    w1c, w1s = w1q if w1q is not None else (None, None)
    w2c, w2s = w2q if w2q is not None else (None, None)
    L.rq_recurrent_prefill(h, S, D, F, w1, w2, w1c, w1s, w2c, w2s, fmt, schedule, steps, eps, workspace,
                           workspace.numel(), stream)
    return h


def pack_nibble_planes(w, scales_f16, stream=None):
    """w int8 [N, K], scales FP16 [N, K/32] -> tiled (hi, lo, scales)."""
    N, K = w.shape
    pb = L.rq_nibble_plane_bytes(N, K)
    hi = _u8((pb,), w.device)
    lo = _u8((pb,), w.device)
    st = torch.empty(L.rq_nibble_scale_bytes(N, K) // 2, dtype=torch.int16, device=w.device)
    L.rq_pack_nibble_planes(w, scales_f16, N, K, hi, lo, st, stream)
    return hi, lo, st


def gemv_nibble_escalate(x, N, planes, flags=None, phase=L.RQ_BOTH, y=None, stream=None, split=True, carry=None):
    """split=False runs every shape unsplit (no workspace).  carry: an FP32
    [B x N] tensor the low pass fills and a later escalation starts from
    (reading only the lo plane); the same split choice on both calls."""
    B, K = x.shape
    hi, lo, st = planes
    if y is None:
        y = torch.empty((B, N), dtype=torch.bfloat16, device=x.device)
    wsb = L.rq_gemv_workspace_bytes(B, N, K) if split else 0
    # the workspace's arrival counters must start at zero (each call leaves them zero)
    ws = torch.zeros((wsb,), dtype=torch.uint8, device=x.device) if wsb else None
    L.rq_gemv_nibble_escalate(x, B, K, N, hi, lo, st, flags, phase, ws, wsb, carry, y, stream)
    return y


def gemv_group(problems, device="cuda"):
    """Plan a grouped GEMV: problems is a list of (x, planes, y) or (x,
    planes, y, carry) with x [B x K] BF16, planes from pack_nibble_planes,
    y [B x N] and the optional FP32 carry [B x N].  Returns (table on the
    device, count, total tiles) for gemv_nibble_escalate_grouped; the table
    refers to the tensors, which must outlive it."""
    arr = (L.RqGemvProblem * len(problems))()
    for i, prob in enumerate(problems):
        x, (hi, lo, st), y = prob[:3]
        carry = prob[3] if len(prob) > 3 else None
        arr[i] = L.RqGemvProblem(x.data_ptr(), hi.data_ptr(), lo.data_ptr() if lo is not None else None,
                                 st.data_ptr(), y.data_ptr(), carry.data_ptr() if carry is not None else None,
                                 y.shape[1], x.shape[1], 0)
    total = L.rq_gemv_group_plan(arr)
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device), len(problems), total


def gemv_nibble_escalate_grouped(table, B, flags=None, phase=L.RQ_BOTH, stream=None):
    dev_table, count, total = table
    L.rq_gemv_nibble_escalate_grouped(dev_table, count, total, B, flags, phase, stream)


def escalation_gate(logits, tau, delta, split=True, stream=None):
    """flags [B] uint8 and stats [B, 2] (entropy, p1 - p2) of logits [B, V];
    split=False runs one workgroup per row (no workspace)."""
    B, V = logits.shape
    flags = _u8((B,), logits.device)
    stats = torch.empty((B, 2), dtype=torch.float32, device=logits.device)
    wsb = L.rq_escalation_gate_workspace_bytes(B, V) if split else 0
    ws = _u8((max(wsb, 16),), logits.device) if wsb else None
    L.rq_escalation_gate(logits, B, V, tau, delta, flags, stats, ws, wsb, stream)
    return flags, stats


def kv_quantize(x, stream=None):
    T, H, D = x.shape
    codes = _u8((T, H, D), x.device)
    scales = torch.empty((T, H, D // 128), dtype=torch.float32, device=x.device)
    L.rq_kv_quantize(x, T, H, D, codes, scales, stream)
    return codes, scales
