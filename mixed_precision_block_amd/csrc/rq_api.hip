// C ABI of librq: argument validation on the host, then kernel launches on
// the caller's stream.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cmath>
#include <utility>
#include <vector>

#include "../../include/rq.h"
#include "rq_internal.h"

namespace {

thread_local char g_err[512] = "";

rq_status fail(rq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rq_status ok() {
  g_err[0] = '\0';
  return RQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A tensor with no elements is never dereferenced, so its pointer may be
// NULL (torch hands out NULL for empty tensors).
bool have(const void* p, bool empty) { return p != nullptr || empty; }

// Device presence, checked after argument validation so that bad arguments
// are reported the same way with or without a GPU.
rq_status need_device() {
  // Queried once per process: the set of visible devices does not change.
  static const std::pair<hipError_t, int> probe = [] {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    return std::make_pair(e, n);
  }();
  if (probe.first != hipSuccess || probe.second <= 0)
    return fail(RQ_ENODEV, "no HIP device visible (%s)", hipGetErrorString(probe.first));
  return RQ_OK;
}

rq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr int64_t kInt32Max = 0x7FFFFFFF;

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

int64_t code_row_bytes(int fmt, int64_t K) { return fmt == RQ_MXFP4 ? K / 2 : K; }

}  // namespace

extern "C" {

int rq_abi_version(void) { return RQ_ABI_VERSION; }

const char* rq_status_str(rq_status s) {
  switch (s) {
    case RQ_OK: return "RQ_OK";
    case RQ_EINVAL: return "RQ_EINVAL";
    case RQ_ESHAPE: return "RQ_ESHAPE";
    case RQ_EALIGN: return "RQ_EALIGN";
    case RQ_EHIP: return "RQ_EHIP";
    case RQ_ENODEV: return "RQ_ENODEV";
  }
  return "RQ_UNKNOWN";
}

const char* rq_last_error(void) { return g_err; }

rq_status rq_quantize(const void* x_bf16, int64_t rows, int64_t K, int fmt, const int32_t* idx, int64_t S,
                      int append, void* codes, uint8_t* scales, void* stream) {
  if (!have(x_bf16, rows == 0) || !have(codes, rows == 0) || !have(scales, rows == 0))
    return fail(RQ_EINVAL, "rq_quantize: null tensor pointer");
  if (fmt != RQ_MXFP4 && fmt != RQ_MXFP8) return fail(RQ_EINVAL, "rq_quantize: fmt must be RQ_MXFP4 or RQ_MXFP8");
  if (append != RQ_APPEND_NONE && append != RQ_APPEND_RESIDUAL && append != RQ_APPEND_COPY)
    return fail(RQ_EINVAL, "rq_quantize: unknown append mode %d", append);
  if (append == RQ_APPEND_NONE && (idx != nullptr || S != 0))
    return fail(RQ_EINVAL, "rq_quantize: RQ_APPEND_NONE needs idx == NULL and S == 0");
  if (append != RQ_APPEND_NONE && (idx == nullptr || S <= 0))
    return fail(RQ_EINVAL, "rq_quantize: an append mode needs idx and S > 0");
  if (rows < 0 || K <= 0 || K % 32 || S < 0 || S % 32)
    return fail(RQ_ESHAPE, "rq_quantize: need rows >= 0, K > 0, K %% 32 == 0, S %% 32 == 0 (rows=%lld K=%lld S=%lld)",
                (long long)rows, (long long)K, (long long)S);
  if (!aligned16(x_bf16) || !aligned16(codes)) return fail(RQ_EALIGN, "rq_quantize: x and codes must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  const int64_t Kp = K + S;
  const int64_t ldc = code_row_bytes(fmt, Kp), lds = Kp / 32;
  hipStream_t st = as_stream(stream);
  hipError_t e;
  if (append == RQ_APPEND_NONE)
    e = rq::launch_quant_rows(fmt, static_cast<const uint16_t*>(x_bf16), rows, K, static_cast<uint8_t*>(codes),
                              scales, ldc, lds, st);
  else
    e = rq::launch_quant_rows_append(fmt, append == RQ_APPEND_RESIDUAL ? 1 : 2, static_cast<const uint16_t*>(x_bf16),
                                     rows, K, idx, S, static_cast<uint8_t*>(codes), scales, st);
  return hip_status(e, "rq_quantize launch");
}

rq_status rq_channel_amax(const void* x_bf16, int64_t rows, int64_t K, uint16_t* amax_bf16, void* stream) {
  if (!have(x_bf16, rows == 0) || !amax_bf16) return fail(RQ_EINVAL, "rq_channel_amax: null pointer");
  if (rows < 0 || K <= 0) return fail(RQ_ESHAPE, "rq_channel_amax: need rows >= 0, K > 0");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_channel_amax(static_cast<const uint16_t*>(x_bf16), rows, K, amax_bf16,
                                            as_stream(stream)),
                    "rq_channel_amax launch");
}

rq_status rq_select_channels(const uint16_t* amax_bf16, int64_t K, int64_t S, int32_t* idx) {
  if (!amax_bf16 || !idx) return fail(RQ_EINVAL, "rq_select_channels: null pointer");
  if (K <= 0 || S < 0 || S > K) return fail(RQ_ESHAPE, "rq_select_channels: need 0 <= S <= K");
  std::vector<int32_t> order(static_cast<size_t>(K));
  for (int64_t k = 0; k < K; ++k) order[k] = static_cast<int32_t>(k);
  // BF16 magnitudes order like their bit patterns (sign cleared).
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return (amax_bf16[a] & 0x7FFF) > (amax_bf16[b] & 0x7FFF);
  });
  std::copy(order.begin(), order.begin() + S, idx);
  return ok();
}

rq_status rq_arc_frontend(const void* x_bf16, int64_t rows, int64_t K, const int32_t* perm, int64_t S, int fmt,
                          int append, int rmsnorm, float eps, void* codes, uint8_t* scales, void* stream) {
  if (!have(x_bf16, rows == 0) || !perm || !have(codes, rows == 0) || !have(scales, rows == 0))
    return fail(RQ_EINVAL, "rq_arc_frontend: null pointer");
  if (fmt != RQ_MXFP4 && fmt != RQ_MXFP8) return fail(RQ_EINVAL, "rq_arc_frontend: fmt must be RQ_MXFP4 or RQ_MXFP8");
  if (append != RQ_APPEND_NONE && append != RQ_APPEND_RESIDUAL && append != RQ_APPEND_COPY)
    return fail(RQ_EINVAL, "rq_arc_frontend: unknown append mode %d", append);
  if ((append == RQ_APPEND_NONE) != (S == 0))
    return fail(RQ_EINVAL, "rq_arc_frontend: RQ_APPEND_NONE exactly when S == 0");
  if (rmsnorm != 0 && rmsnorm != 1) return fail(RQ_EINVAL, "rq_arc_frontend: rmsnorm must be 0 or 1");
  if (rmsnorm && !(eps >= 0.0f && eps < INFINITY)) return fail(RQ_EINVAL, "rq_arc_frontend: eps must be finite and >= 0");
  if (rows < 0 || rows > kInt32Max || K <= 0 || K % 32 || K > 16384 || S < 0 || S % 32 || S > K)
    return fail(RQ_ESHAPE, "rq_arc_frontend: need 0 <= rows < 2^31, 0 < K <= 16384, K %% 32 == 0, "
                           "0 <= S <= K, S %% 32 == 0 (rows=%lld K=%lld S=%lld)",
                (long long)rows, (long long)K, (long long)S);
  if (!aligned16(x_bf16) || !aligned16(perm) || !aligned16(codes))
    return fail(RQ_EALIGN, "rq_arc_frontend: x, perm and codes must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_arc_frontend(fmt, append == RQ_APPEND_RESIDUAL ? 1 : (append == RQ_APPEND_COPY ? 2 : 0),
                                            rmsnorm == 1, static_cast<const uint16_t*>(x_bf16), rows, K, perm, S,
                                            eps, static_cast<uint8_t*>(codes), scales, as_stream(stream)),
                    "rq_arc_frontend launch");
}

rq_status rq_rmsnorm(const void* h_bf16, int64_t rows, int64_t D, float eps, void* out_bf16, void* stream) {
  if (!have(h_bf16, rows == 0) || !have(out_bf16, rows == 0)) return fail(RQ_EINVAL, "rq_rmsnorm: null pointer");
  if (!(eps >= 0.0f && eps < INFINITY)) return fail(RQ_EINVAL, "rq_rmsnorm: eps must be finite and >= 0");
  if (rows < 0 || rows > kInt32Max || D <= 0 || D % 8)
    return fail(RQ_ESHAPE, "rq_rmsnorm: need 0 <= rows < 2^31, D > 0, D %% 8 == 0");
  if (!aligned16(h_bf16) || !aligned16(out_bf16)) return fail(RQ_EALIGN, "rq_rmsnorm: h and out must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_rmsnorm(RQ_BF16, static_cast<const uint16_t*>(h_bf16), rows, D, eps, out_bf16, nullptr,
                                       as_stream(stream)),
                    "rq_rmsnorm launch");
}

rq_status rq_gemm(int fmt, const void* a, const uint8_t* a_scales, const void* w, const uint8_t* w_scales,
                  int64_t M, int64_t N, int64_t K, int out, void* y, void* stream) {
  if (!have(a, M == 0) || !have(w, N == 0) || !have(y, M == 0 || N == 0))
    return fail(RQ_EINVAL, "rq_gemm: null tensor pointer");
  if (fmt != RQ_MXFP4 && fmt != RQ_MXFP8 && fmt != RQ_BF16 && fmt != RQ_MXFP8_F8MFMA)
    return fail(RQ_EINVAL, "rq_gemm: unknown fmt %d", fmt);
  if (fmt == RQ_BF16 && (a_scales || w_scales)) return fail(RQ_EINVAL, "rq_gemm: RQ_BF16 takes no scales");
  if (fmt != RQ_BF16 && (!have(a_scales, M == 0) || !have(w_scales, N == 0)))
    return fail(RQ_EINVAL, "rq_gemm: MX formats need scales");
  if (out != RQ_OUT_BF16 && out != RQ_OUT_F32) return fail(RQ_EINVAL, "rq_gemm: unknown out %d", out);
  if (M < 0 || N < 0 || K <= 0 || K % 32 || M > kInt32Max || N > kInt32Max || K > kInt32Max)
    return fail(RQ_ESHAPE, "rq_gemm: need 0 <= M, N < 2^31 and 0 < K < 2^31 with K %% 32 == 0");
  if (!aligned16(a) || !aligned16(w) || !aligned16(y)) return fail(RQ_EALIGN, "rq_gemm: a, w, y must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_gemm(fmt, out == RQ_OUT_F32 ? rq::kEpiStoreF32 : rq::kEpiStoreBf16, a, a_scales, w,
                                    w_scales, M, N, K, y, as_stream(stream)),
                    "rq_gemm launch");
}

size_t rq_gemm_arc_workspace_bytes(int64_t M, int64_t K, int64_t S) {
  if (M < 0 || K < 0 || S < 0) return 0;
  const int64_t Kp = K + S;
  return round256(static_cast<size_t>(M * (Kp / 2))) + round256(static_cast<size_t>(M * (Kp / 32)));
}

rq_status rq_gemm_arc(const void* a_bf16, int64_t M, int64_t K, const int32_t* idx, int64_t S, const void* w_aug,
                      const uint8_t* w_aug_scales, int64_t N, void* workspace, size_t ws_bytes, int out, void* y,
                      void* stream) {
  if (!have(a_bf16, M == 0) || !idx || !have(w_aug, N == 0) || !have(w_aug_scales, N == 0) ||
      !have(workspace, M == 0) || !have(y, M == 0 || N == 0))
    return fail(RQ_EINVAL, "rq_gemm_arc: null pointer");
  if (out != RQ_OUT_BF16 && out != RQ_OUT_F32) return fail(RQ_EINVAL, "rq_gemm_arc: unknown out %d", out);
  if (M < 0 || N < 0 || K <= 0 || K % 32 || S <= 0 || S % 32 || M > kInt32Max || N > kInt32Max ||
      K + S > kInt32Max)
    return fail(RQ_ESHAPE, "rq_gemm_arc: need K %% 32 == 0, S > 0, S %% 32 == 0, sizes < 2^31");
  if (ws_bytes < rq_gemm_arc_workspace_bytes(M, K, S))
    return fail(RQ_ESHAPE, "rq_gemm_arc: workspace %zu < %zu bytes", ws_bytes, rq_gemm_arc_workspace_bytes(M, K, S));
  if (!aligned16(a_bf16) || !aligned16(w_aug) || !aligned16(workspace) || !aligned16(y))
    return fail(RQ_EALIGN, "rq_gemm_arc: a, w_aug, workspace, y must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  const int64_t Kp = K + S;
  uint8_t* codes = static_cast<uint8_t*>(workspace);
  uint8_t* scales = codes + round256(static_cast<size_t>(M * (Kp / 2)));
  hipStream_t st = as_stream(stream);
  hipError_t e = rq::launch_quant_rows_append(RQ_MXFP4, 1, static_cast<const uint16_t*>(a_bf16), M, K, idx, S, codes,
                                              scales, st);
  if (e == hipSuccess)
    e = rq::launch_gemm(RQ_MXFP4, out == RQ_OUT_F32 ? rq::kEpiStoreF32 : rq::kEpiStoreBf16, codes, scales, w_aug,
                        w_aug_scales, M, N, Kp, y, st);
  return hip_status(e, "rq_gemm_arc launch");
}

// Workspace of the recurrent prefill: [n codes or BF16 | n scales | u BF16 |
// u codes | u scales], each 256-byte aligned.
size_t rq_recurrent_prefill_workspace_bytes(int64_t S, int64_t D, int64_t F, int fmt) {
  (void)fmt;
  if (S < 0 || D < 0 || F < 0) return 0;
  const size_t s = static_cast<size_t>(S), d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  return round256(s * d * 2) + round256(s * (d / 32)) + round256(s * f * 2) + round256(s * f) +
         round256(s * (f / 32));
}

rq_status rq_recurrent_prefill(void* h_bf16, int64_t S, int64_t D, int64_t F, const void* w1_bf16,
                               const void* w2_bf16, const void* w1_q, const uint8_t* w1_s, const void* w2_q,
                               const uint8_t* w2_s, int fmt, uint64_t schedule, int steps, float eps,
                               void* workspace, size_t ws_bytes, void* stream) {
  if (!have(h_bf16, S == 0) || !have(workspace, S == 0))
    return fail(RQ_EINVAL, "rq_recurrent_prefill: null h or workspace");
  if (fmt != RQ_MXFP4 && fmt != RQ_MXFP8 && fmt != RQ_MXFP8_F8MFMA)
    return fail(RQ_EINVAL, "rq_recurrent_prefill: fmt must be RQ_MXFP4, RQ_MXFP8 or RQ_MXFP8_F8MFMA");
  if (steps < 1 || steps > 64) return fail(RQ_ESHAPE, "rq_recurrent_prefill: steps must be in [1, 64]");
  const uint64_t used = steps == 64 ? ~0ull : ((1ull << steps) - 1);
  const bool any_q = (schedule & used) != 0, any_bf16 = (~schedule & used) != 0;
  if (any_q && (!w1_q || !w1_s || !w2_q || !w2_s))
    return fail(RQ_EINVAL, "rq_recurrent_prefill: quantized steps need w1_q, w1_s, w2_q, w2_s");
  if (any_bf16 && (!w1_bf16 || !w2_bf16)) return fail(RQ_EINVAL, "rq_recurrent_prefill: BF16 steps need w1/w2 BF16");
  if (!(eps >= 0.0f)) return fail(RQ_EINVAL, "rq_recurrent_prefill: eps must be >= 0");
  if (S < 0 || D <= 0 || F <= 0 || D % 32 || F % 32 || S > kInt32Max || D > kInt32Max || F > kInt32Max)
    return fail(RQ_ESHAPE, "rq_recurrent_prefill: need D, F > 0 multiples of 32, sizes < 2^31");
  const size_t need = rq_recurrent_prefill_workspace_bytes(S, D, F, fmt);
  if (ws_bytes < need) return fail(RQ_ESHAPE, "rq_recurrent_prefill: workspace %zu < %zu bytes", ws_bytes, need);
  const void* ptrs[] = {h_bf16, w1_bf16, w2_bf16, w1_q, w2_q, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(RQ_EALIGN, "rq_recurrent_prefill: tensors must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;

  const size_t sz = static_cast<size_t>(S), dz = static_cast<size_t>(D), fz = static_cast<size_t>(F);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* n_buf = base;
  uint8_t* n_sc = n_buf + round256(sz * dz * 2);
  uint8_t* u_buf = n_sc + round256(sz * (dz / 32));
  uint8_t* u_codes = u_buf + round256(sz * fz * 2);
  uint8_t* u_sc = u_codes + round256(sz * fz);
  uint16_t* h = static_cast<uint16_t*>(h_bf16);
  hipStream_t st = as_stream(stream);
  // the codes n and u are quantized to (MXFP8 for both MXFP8 GEMM forms)
  const int qfmt = fmt == RQ_MXFP8_F8MFMA ? RQ_MXFP8 : fmt;
  // shapes the pipelined GEMM takes quantize u in W1's epilogue (the same
  // codes as the separate pass); the others go through u in BF16
  const bool fused_u = rq::gemm_pipe_supported(fmt, S, F, D);
  for (int t = 1; t <= steps; ++t) {
    const bool q = (schedule >> (t - 1)) & 1ull;
    hipError_t e;
    if (q) {
      e = rq::launch_rmsnorm(qfmt, h, S, D, eps, n_buf, n_sc, st);
      if (e == hipSuccess) {
        if (fused_u) {
          // SiLU and the block quantization of u in W1's epilogue
          e = rq::launch_gemm_silu_quant(fmt, n_buf, n_sc, w1_q, w1_s, S, F, D, u_codes, u_sc, st);
        } else {
          e = rq::launch_gemm(fmt, rq::kEpiSiluBf16, n_buf, n_sc, w1_q, w1_s, S, F, D, u_buf, st);
          if (e == hipSuccess)
            e = rq::launch_quant_rows(qfmt, reinterpret_cast<const uint16_t*>(u_buf), S, F, u_codes, u_sc,
                                      code_row_bytes(qfmt, F), F / 32, st);
        }
      }
      if (e == hipSuccess) e = rq::launch_gemm(fmt, rq::kEpiResAddBf16, u_codes, u_sc, w2_q, w2_s, S, D, F, h, st);
    } else {
      e = rq::launch_rmsnorm(RQ_BF16, h, S, D, eps, n_buf, nullptr, st);
      if (e == hipSuccess) e = rq::launch_gemm(RQ_BF16, rq::kEpiSiluBf16, n_buf, nullptr, w1_bf16, nullptr, S, F, D, u_buf, st);
      if (e == hipSuccess) e = rq::launch_gemm(RQ_BF16, rq::kEpiResAddBf16, u_buf, nullptr, w2_bf16, nullptr, S, D, F, h, st);
    }
    if (e != hipSuccess) return hip_status(e, "rq_recurrent_prefill launch");
  }
  return ok();
}

size_t rq_nibble_plane_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return static_cast<size_t>((N + 63) / 64 * 64) * static_cast<size_t>(K / 2);
}

size_t rq_nibble_scale_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return static_cast<size_t>((N + 63) / 64 * 64) * static_cast<size_t>(K / 32) * 2;
}

rq_status rq_pack_nibble_planes(const int8_t* w, const uint16_t* scales_f16, int64_t N, int64_t K, uint8_t* hi,
                                uint8_t* lo, uint16_t* scales_tiled, void* stream) {
  if (!have(w, N == 0) || !have(scales_f16, N == 0) || !have(hi, N == 0) || !have(lo, N == 0) ||
      !have(scales_tiled, N == 0))
    return fail(RQ_EINVAL, "rq_pack_nibble_planes: null pointer");
  if (N < 0 || K <= 0 || K % 32 || N > kInt32Max || K > kInt32Max)
    return fail(RQ_ESHAPE, "rq_pack_nibble_planes: need K > 0, K %% 32 == 0");
  if (!aligned16(hi) || !aligned16(lo)) return fail(RQ_EALIGN, "rq_pack_nibble_planes: planes must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_pack_nibble_planes(w, scales_f16, N, K, hi, lo, scales_tiled, as_stream(stream)),
                    "rq_pack_nibble_planes launch");
}

size_t rq_gemv_workspace_bytes(int64_t B, int64_t N, int64_t K) {
  if (B < 1 || B > 16 || N <= 0 || K <= 0 || K % 32) return 0;
  return rq::gemv_workspace_bytes(B, N, K);
}

rq_status rq_gemv_nibble_escalate(const void* x_bf16, int64_t B, int64_t K, int64_t N, const uint8_t* w_hi,
                                  const uint8_t* w_lo, const uint16_t* scales_tiled, const uint8_t* flags, int phase,
                                  void* workspace, size_t ws_bytes, float* y_f32, void* y_bf16, void* stream) {
  // the hi plane is read by the low pass and by an escalation without a carry
  const bool need_hi = (phase & RQ_LOW) || !y_f32;
  if (!x_bf16 || (need_hi && !have(w_hi, N == 0)) || !have(scales_tiled, N == 0) || !have(y_bf16, N == 0))
    return fail(RQ_EINVAL, "rq_gemv_nibble_escalate: null pointer");
  if (phase != RQ_LOW && phase != RQ_ESCALATE && phase != RQ_BOTH)
    return fail(RQ_EINVAL, "rq_gemv_nibble_escalate: unknown phase %d", phase);
  if ((phase & RQ_ESCALATE) && (!have(w_lo, N == 0) || !flags))
    return fail(RQ_EINVAL, "rq_gemv_nibble_escalate: escalation needs w_lo and flags");
  if (B < 1 || B > 16) return fail(RQ_ESHAPE, "rq_gemv_nibble_escalate: B must be in [1, 16]");
  if (N < 0 || K <= 0 || K % 32 || N > kInt32Max || K > kInt32Max)
    return fail(RQ_ESHAPE, "rq_gemv_nibble_escalate: need K > 0, K %% 32 == 0");
  if (!aligned16(x_bf16) || !aligned16(w_hi) || (w_lo && !aligned16(w_lo)))
    return fail(RQ_EALIGN, "rq_gemv_nibble_escalate: x and planes must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(y_f32) & 3u) != 0)
    return fail(RQ_EALIGN, "rq_gemv_nibble_escalate: y_f32 must be 4-byte aligned");
  if (workspace && !aligned16(workspace)) return fail(RQ_EALIGN, "rq_gemv_nibble_escalate: workspace must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  hipStream_t st = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint16_t* y = static_cast<uint16_t*>(y_bf16);
  hipError_t e = hipSuccess;
  const size_t wsb = workspace ? ws_bytes : 0;
  if (phase & RQ_LOW) e = rq::launch_gemv_low(x, B, K, N, w_hi, scales_tiled, y, y_f32, workspace, wsb, st);
  if (e == hipSuccess && (phase & RQ_ESCALATE))
    e = rq::launch_gemv_escalate(x, B, K, N, w_hi, w_lo, scales_tiled, flags, y, y_f32, workspace, wsb, st);
  return hip_status(e, "rq_gemv_nibble_escalate launch");
}

int64_t rq_gemv_group_plan(rq_gemv_problem* problems, int count) {
  if (!problems || count < 1) {
    fail(RQ_EINVAL, "rq_gemv_group_plan: need problems and count >= 1");
    return -1;
  }
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    rq_gemv_problem& p = problems[i];
    if (!p.x_bf16 || !p.w_hi || !p.scales_tiled || !p.y_bf16) {
      fail(RQ_EINVAL, "rq_gemv_group_plan: problem %d has a null pointer", i);
      return -1;
    }
    if (p.N <= 0 || p.K <= 0 || p.K % 32 || p.N > kInt32Max || p.K > kInt32Max) {
      fail(RQ_ESHAPE, "rq_gemv_group_plan: problem %d needs N > 0, K > 0, K %% 32 == 0", i);
      return -1;
    }
    if (!aligned16(p.x_bf16) || !aligned16(p.w_hi) || (p.w_lo && !aligned16(p.w_lo))) {
      fail(RQ_EALIGN, "rq_gemv_group_plan: problem %d: x and planes must be 16-byte aligned", i);
      return -1;
    }
    if ((reinterpret_cast<uintptr_t>(p.y_f32) & 3u) != 0) {
      fail(RQ_EALIGN, "rq_gemv_group_plan: problem %d: y_f32 must be 4-byte aligned", i);
      return -1;
    }
    p.tile_start = tiles;
    tiles += (p.N + 63) / 64;
  }
  if (tiles > kInt32Max) {
    fail(RQ_ESHAPE, "rq_gemv_group_plan: too many tiles");
    return -1;
  }
  ok();
  return tiles;
}

rq_status rq_gemv_nibble_escalate_grouped(const rq_gemv_problem* problems_dev, int count, int64_t total_tiles,
                                          int64_t B, const uint8_t* flags, int phase, void* stream) {
  if (!problems_dev) return fail(RQ_EINVAL, "rq_gemv_nibble_escalate_grouped: null problem table");
  if (phase != RQ_LOW && phase != RQ_ESCALATE && phase != RQ_BOTH)
    return fail(RQ_EINVAL, "rq_gemv_nibble_escalate_grouped: unknown phase %d", phase);
  if ((phase & RQ_ESCALATE) && !flags)
    return fail(RQ_EINVAL, "rq_gemv_nibble_escalate_grouped: escalation needs flags");
  if (count < 1 || total_tiles < 1 || total_tiles > kInt32Max)
    return fail(RQ_ESHAPE, "rq_gemv_nibble_escalate_grouped: need count >= 1 and a planned tile total");
  if (B < 1 || B > 16) return fail(RQ_ESHAPE, "rq_gemv_nibble_escalate_grouped: B must be in [1, 16]");
  if (!aligned16(problems_dev)) return fail(RQ_EALIGN, "rq_gemv_nibble_escalate_grouped: table must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_gemv_grouped(problems_dev, count, total_tiles, B, flags, phase, as_stream(stream)),
                    "rq_gemv_nibble_escalate_grouped launch");
}

size_t rq_escalation_gate_workspace_bytes(int64_t B, int64_t V) { return rq::gate_workspace_bytes(B, V); }

rq_status rq_escalation_gate(const void* logits_bf16, int64_t B, int64_t V, float tau, float delta, uint8_t* flags,
                             float* stats, void* workspace, size_t ws_bytes, void* stream) {
  if (!logits_bf16 || !flags) return fail(RQ_EINVAL, "rq_escalation_gate: null pointer");
  if (B < 1 || B > 16 || V < 2 || V > kInt32Max) return fail(RQ_ESHAPE, "rq_escalation_gate: need B in [1, 16] and V >= 2");
  if ((reinterpret_cast<uintptr_t>(logits_bf16) & 1u) != 0)
    return fail(RQ_EALIGN, "rq_escalation_gate: logits must be 2-byte aligned");
  if ((reinterpret_cast<uintptr_t>(stats) & 3u) != 0) return fail(RQ_EALIGN, "rq_escalation_gate: stats must be 4-byte aligned");
  if (workspace && !aligned16(workspace)) return fail(RQ_EALIGN, "rq_escalation_gate: workspace must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_gate(static_cast<const uint16_t*>(logits_bf16), B, V, tau, delta, flags, stats,
                                    workspace, ws_bytes, as_stream(stream)),
                    "rq_escalation_gate launch");
}

rq_status rq_escalation_gate_noalloc(const void* logits_bf16, int64_t B, int64_t V, float tau, float delta,
                                     uint8_t* flags, float* stats, void* stream) {
  if (!logits_bf16 || !flags) return fail(RQ_EINVAL, "rq_escalation_gate_noalloc: null pointer");
  if (B < 1 || B > 16 || V < 2 || V > kInt32Max)
    return fail(RQ_ESHAPE, "rq_escalation_gate_noalloc: need B in [1, 16] and V >= 2");
  if ((reinterpret_cast<uintptr_t>(logits_bf16) & 1u) != 0)
    return fail(RQ_EALIGN, "rq_escalation_gate_noalloc: logits must be 2-byte aligned");
  if ((reinterpret_cast<uintptr_t>(stats) & 3u) != 0)
    return fail(RQ_EALIGN, "rq_escalation_gate_noalloc: stats must be 4-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (hipError_t e = rq::gate_scratch(&ws, &ws_bytes); e != hipSuccess)
    return fail(RQ_EHIP, "rq_escalation_gate_noalloc: scratch lookup: %s", hipGetErrorString(e));
  const size_t need = rq::gate_workspace_bytes(B, V);
  if (need > ws_bytes)
    return fail(RQ_ESHAPE, "rq_escalation_gate_noalloc: needs %zu bytes of scratch, the static scratch holds %zu",
                need, ws_bytes);
  return hip_status(rq::launch_gate(static_cast<const uint16_t*>(logits_bf16), B, V, tau, delta, flags, stats, ws,
                                    ws_bytes, as_stream(stream)),
                    "rq_escalation_gate_noalloc launch");
}

rq_status rq_kv_quantize(const void* x_bf16, int64_t T, int64_t H, int64_t D, uint8_t* codes, float* scales,
                         void* stream) {
  const bool kv_empty = T == 0 || H == 0;
  if (!have(x_bf16, kv_empty) || !have(codes, kv_empty) || !have(scales, kv_empty))
    return fail(RQ_EINVAL, "rq_kv_quantize: null pointer");
  if (T < 0 || H < 0 || D <= 0 || D % 128) return fail(RQ_ESHAPE, "rq_kv_quantize: need D > 0, D %% 128 == 0");
  if (!aligned16(x_bf16) || !aligned16(codes)) return fail(RQ_EALIGN, "rq_kv_quantize: x and codes must be 16-byte aligned");
  if (rq_status s = need_device(); s != RQ_OK) return s;
  return hip_status(rq::launch_kv_quant(static_cast<const uint16_t*>(x_bf16), T, H, D, codes, scales,
                                        as_stream(stream)),
                    "rq_kv_quantize launch");
}

}  // extern "C"
