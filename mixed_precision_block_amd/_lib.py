"""ctypes binding of librq (include/rq.h): argument marshalling only.

Each rq_* function below has the C function's name and argument order.
Tensor arguments accept a torch tensor (its data_ptr() is passed), a plain
integer address, or None for NULL.  `stream` defaults to torch's current
stream on the current device.  A non-OK status raises RQError carrying the
status and the library's error text.  Nothing here computes: every step of
the path runs in the HIP kernels of librq.so, and a missing library raises
instead of falling back to anything else.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librq.so")

RQ_OK, RQ_EINVAL, RQ_ESHAPE, RQ_EALIGN, RQ_EHIP, RQ_ENODEV = range(6)
RQ_MXFP4, RQ_MXFP8, RQ_BF16, RQ_MXFP8_F8MFMA = 1, 2, 3, 4
RQ_APPEND_NONE, RQ_APPEND_RESIDUAL, RQ_APPEND_COPY = 0, 1, 2
RQ_OUT_BF16, RQ_OUT_F32 = 0, 1
RQ_LOW, RQ_ESCALATE, RQ_BOTH = 1, 2, 3


class RQError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name


class RqGemvProblem(ctypes.Structure):
    """rq_gemv_problem: one problem of a grouped GEMV launch (include/rq.h)."""
    _fields_ = [("x_bf16", ctypes.c_void_p), ("w_hi", ctypes.c_void_p), ("w_lo", ctypes.c_void_p),
                ("scales_tiled", ctypes.c_void_p), ("y_bf16", ctypes.c_void_p), ("y_f32", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("tile_start", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_U64 = ctypes.c_uint64

# name -> (restype, argtypes)
_SIGNATURES = {
    "rq_abi_version": (_INT, []),
    "rq_status_str": (ctypes.c_char_p, [_INT]),
    "rq_last_error": (ctypes.c_char_p, []),
    "rq_quantize": (_INT, [_P, _I64, _I64, _INT, _P, _I64, _INT, _P, _P, _P]),
    "rq_channel_amax": (_INT, [_P, _I64, _I64, _P, _P]),
    "rq_select_channels": (_INT, [_P, _I64, _I64, _P]),
    "rq_arc_frontend": (_INT, [_P, _I64, _I64, _P, _I64, _INT, _INT, _INT, _F, _P, _P, _P]),
    "rq_rmsnorm": (_INT, [_P, _I64, _I64, _F, _P, _P]),
    "rq_gemm": (_INT, [_INT, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _P]),
    "rq_gemm_arc_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "rq_gemm_arc": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _I64, _P, _SZ, _INT, _P, _P]),
    "rq_recurrent_prefill_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "rq_recurrent_prefill": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _INT, _U64, _INT, _F,
                                    _P, _SZ, _P]),
    "rq_nibble_plane_bytes": (_SZ, [_I64, _I64]),
    "rq_nibble_scale_bytes": (_SZ, [_I64, _I64]),
    "rq_pack_nibble_planes": (_INT, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "rq_gemv_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "rq_gemv_nibble_escalate": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _INT, _P, _SZ, _P, _P, _P]),
    "rq_gemv_group_plan": (_I64, [ctypes.POINTER(RqGemvProblem), _INT]),
    "rq_gemv_nibble_escalate_grouped": (_INT, [_P, _INT, _I64, _I64, _P, _INT, _P]),
    "rq_escalation_gate_workspace_bytes": (_SZ, [_I64, _I64]),
    "rq_escalation_gate": (_INT, [_P, _I64, _I64, _F, _F, _P, _P, _P, _SZ, _P]),
    "rq_escalation_gate_noalloc": (_INT, [_P, _I64, _I64, _F, _F, _P, _P, _P]),
    "rq_kv_quantize": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P]),
}

_lib = None

# The RQ_ABI_VERSION these signatures and RqGemvProblem follow (include/rq.h).
ABI_VERSION = 5


def lib():
    """The loaded librq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librq.so not found at {LIB_PATH}; build it with "
                               "`python -m mixed_precision_block_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.rq_abi_version() != ABI_VERSION:
            raise RuntimeError(f"librq.so has ABI version {handle.rq_abi_version()}, this binding expects "
                               f"{ABI_VERSION}; rebuild it with `python -m mixed_precision_block_amd.build`")
        _lib = handle
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(name, status):
    if status != RQ_OK:
        L = lib()
        raise RQError(status, name, f"{L.rq_status_str(status).decode()}: {L.rq_last_error().decode()}")


def rq_abi_version():
    return lib().rq_abi_version()


def rq_quantize(x, rows, K, fmt, idx, S, append, codes, scales, stream=None):
    _check("rq_quantize", lib().rq_quantize(_ptr(x), rows, K, fmt, _ptr(idx), S, append, _ptr(codes),
                                           _ptr(scales), _stream(stream)))


def rq_channel_amax(x, rows, K, amax, stream=None):
    _check("rq_channel_amax", lib().rq_channel_amax(_ptr(x), rows, K, _ptr(amax), _stream(stream)))


def rq_select_channels(amax_host, K, S, idx_host):
    """amax_host / idx_host: CPU tensors or host addresses."""
    _check("rq_select_channels", lib().rq_select_channels(_ptr(amax_host), K, S, _ptr(idx_host)))


def rq_arc_frontend(x, rows, K, perm, S, fmt, append, rmsnorm, eps, codes, scales, stream=None):
    _check("rq_arc_frontend", lib().rq_arc_frontend(_ptr(x), rows, K, _ptr(perm), S, fmt, append, rmsnorm, eps,
                                                    _ptr(codes), _ptr(scales), _stream(stream)))


def rq_rmsnorm(h, rows, D, eps, out, stream=None):
    _check("rq_rmsnorm", lib().rq_rmsnorm(_ptr(h), rows, D, eps, _ptr(out), _stream(stream)))


def rq_gemm(fmt, a, a_scales, w, w_scales, M, N, K, out, y, stream=None):
    _check("rq_gemm", lib().rq_gemm(fmt, _ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), M, N, K, out,
                                    _ptr(y), _stream(stream)))


def rq_gemm_arc_workspace_bytes(M, K, S):
    return lib().rq_gemm_arc_workspace_bytes(M, K, S)


def rq_gemm_arc(a, M, K, idx, S, w_aug, w_aug_scales, N, workspace, ws_bytes, out, y, stream=None):
    _check("rq_gemm_arc", lib().rq_gemm_arc(_ptr(a), M, K, _ptr(idx), S, _ptr(w_aug), _ptr(w_aug_scales), N,
                                            _ptr(workspace), ws_bytes, out, _ptr(y), _stream(stream)))


def rq_recurrent_prefill_workspace_bytes(S, D, F, fmt):
    return lib().rq_recurrent_prefill_workspace_bytes(S, D, F, fmt)


def rq_recurrent_prefill(h, S, D, F, w1, w2, w1_q, w1_s, w2_q, w2_s, fmt, schedule, steps, eps, workspace,
                         ws_bytes, stream=None):
    _check("rq_recurrent_prefill",
           lib().rq_recurrent_prefill(_ptr(h), S, D, F, _ptr(w1), _ptr(w2), _ptr(w1_q), _ptr(w1_s), _ptr(w2_q),
                                      _ptr(w2_s), fmt, schedule, steps, eps, _ptr(workspace), ws_bytes,
                                      _stream(stream)))


def rq_nibble_plane_bytes(N, K):
    return lib().rq_nibble_plane_bytes(N, K)


def rq_nibble_scale_bytes(N, K):
    return lib().rq_nibble_scale_bytes(N, K)


def rq_pack_nibble_planes(w, scales, N, K, hi, lo, scales_tiled, stream=None):
    _check("rq_pack_nibble_planes", lib().rq_pack_nibble_planes(_ptr(w), _ptr(scales), N, K, _ptr(hi), _ptr(lo),
                                                                _ptr(scales_tiled), _stream(stream)))


def rq_gemv_workspace_bytes(B, N, K):
    return lib().rq_gemv_workspace_bytes(B, N, K)


def rq_gemv_nibble_escalate(x, B, K, N, w_hi, w_lo, scales_tiled, flags, phase, workspace, ws_bytes, y_f32, y,
                            stream=None):
    _check("rq_gemv_nibble_escalate",
           lib().rq_gemv_nibble_escalate(_ptr(x), B, K, N, _ptr(w_hi), _ptr(w_lo), _ptr(scales_tiled), _ptr(flags),
                                         phase, _ptr(workspace), ws_bytes, _ptr(y_f32), _ptr(y), _stream(stream)))


def rq_gemv_group_plan(problems):
    """problems: a ctypes array of RqGemvProblem (filled in place); returns
    the total tile count or raises."""
    total = lib().rq_gemv_group_plan(problems, len(problems))
    if total < 0:
        raise RQError(RQ_EINVAL, "rq_gemv_group_plan", lib().rq_last_error().decode())
    return total


def rq_gemv_nibble_escalate_grouped(problems_dev, count, total_tiles, B, flags, phase, stream=None):
    _check("rq_gemv_nibble_escalate_grouped",
           lib().rq_gemv_nibble_escalate_grouped(_ptr(problems_dev), count, total_tiles, B, _ptr(flags), phase,
                                                 _stream(stream)))


def rq_escalation_gate_workspace_bytes(B, V):
    return lib().rq_escalation_gate_workspace_bytes(B, V)


def rq_escalation_gate(logits, B, V, tau, delta, flags, stats, workspace, ws_bytes, stream=None):
    _check("rq_escalation_gate", lib().rq_escalation_gate(_ptr(logits), B, V, tau, delta, _ptr(flags),
                                                          _ptr(stats), _ptr(workspace), ws_bytes,
                                                          _stream(stream)))


def rq_escalation_gate_noalloc(logits, B, V, tau, delta, flags, stats, stream=None):
    _check("rq_escalation_gate_noalloc", lib().rq_escalation_gate_noalloc(_ptr(logits), B, V, tau, delta,
                                                                          _ptr(flags), _ptr(stats),
                                                                          _stream(stream)))


def rq_kv_quantize(x, T, H, D, codes, scales, stream=None):
    _check("rq_kv_quantize", lib().rq_kv_quantize(_ptr(x), T, H, D, _ptr(codes), _ptr(scales), _stream(stream)))
