// Internal launch interface between the C ABI layer (rq_api.hip) and the
// kernel translation units.  Every launcher enqueues on `stream` and
// returns hipGetLastError() of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

struct rq_gemv_problem;  // include/rq.h

namespace rq {

// GEMM epilogues.  Y is [M x N] row-major.
enum Epilogue {
  kEpiStoreBf16 = 0,  // y = bf16(acc)
  kEpiStoreF32 = 1,   // y = acc
  kEpiSiluBf16 = 2,   // y = bf16(SiLU(bf16(acc)))
  kEpiResAddBf16 = 3, // y = bf16(y + bf16(acc))   (in place)
  kEpiSiluQuant = 4   // u = bf16(SiLU(bf16(acc))), stored as the GEMM's MX format: codes y, scales ys
};

// fmt: 1 = MXFP4, 2 = MXFP8, 3 = BF16 (scale pointers ignored).  Picks the
// pipelined kernel when it applies, else the general one.
hipError_t launch_gemm(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                       const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                       hipStream_t stream);
// The general kernel (any K % 32 == 0) and the pipelined one (K % 128 == 0
// for MXFP4 / MXFP8, K % 32 == 0 for BF16).
hipError_t launch_gemm_basic(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                             const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                             hipStream_t stream);
bool gemm_pipe_supported(int fmt, int64_t M, int64_t N, int64_t K);
// y = SiLU(A W^T) rounded to BF16 and block-quantized, in one launch: codes
// [M x N] in fmt's layout (row stride N/2 or N bytes) and scales [M x N/32].
// MXFP4 / MXFP8 only; needs gemm_pipe_supported and N % 32 == 0, else
// returns hipErrorInvalidValue without launching.
hipError_t launch_gemm_silu_quant(int fmt, const void* a, const uint8_t* a_scales, const void* w,
                                  const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, uint8_t* codes,
                                  uint8_t* scales, hipStream_t stream);
hipError_t launch_gemm_pipe(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                            const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                            hipStream_t stream);

// Primary block quantization of rows [rows x K] into codes/scales whose
// row strides are ldc_bytes / lds_bytes (room for appended columns).
hipError_t launch_quant_rows(int fmt, const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                             uint8_t* scales, int64_t ldc_bytes, int64_t lds_bytes,
                             hipStream_t stream);
// Appended columns K..K+S-1 (mode 1 residual, 2 copy); reads the primary
// scales of the same rows for the residual.
hipError_t launch_quant_append(int fmt, int mode, const uint16_t* x, int64_t rows, int64_t K,
                               const int32_t* idx, int64_t S, uint8_t* codes, uint8_t* scales,
                               int64_t ldc_bytes, int64_t lds_bytes, hipStream_t stream);
// Primary quantization with appended columns (mode 1 residual, 2 copy) in
// one pass over each row, codes [rows x (K+S)] (FP4 packed) and scales
// [rows x (K+S)/32]; S == 0 is plain quantization.  Falls back to the two
// passes above for S > 2048 or K > 16384.
hipError_t launch_quant_rows_append(int fmt, int mode, const uint16_t* x, int64_t rows, int64_t K,
                                    const int32_t* idx, int64_t S, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream);
// Fused front end: optional RMSNorm (eps, no gain), reorder by perm,
// primary block quantization over K, and for positions 0..S-1 an appended
// block (mode 1 residual, 2 copy; S == 0 for none).  K <= 16384 (the row
// is staged in LDS).
hipError_t launch_arc_frontend(int fmt, int mode, bool norm, const uint16_t* x, int64_t rows, int64_t K,
                               const int32_t* perm, int64_t S, float eps, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream);
hipError_t launch_channel_amax(const uint16_t* x, int64_t rows, int64_t K, uint16_t* amax,
                               hipStream_t stream);

// RMSNorm (eps, no gain) of rows [rows x D]: to BF16 (fmt == 3) or fused
// with block quantization to MX codes/scales (fmt 1/2).
hipError_t launch_rmsnorm(int fmt, const uint16_t* h, int64_t rows, int64_t D, float eps,
                          void* out, uint8_t* out_scales, hipStream_t stream);

// Nibble planes and decode GEMV.
hipError_t launch_pack_nibble_planes(const int8_t* w, const uint16_t* scales, int64_t N, int64_t K,
                                     uint8_t* hi, uint8_t* lo, uint16_t* scales_tiled,
                                     hipStream_t stream);
// Workspace (FP32 partials of split-K launches) of rq_gemv_nibble_escalate;
// 0 when the shape needs no split.  With less workspace than this the
// kernels run unsplit.
size_t gemv_workspace_bytes(int64_t B, int64_t N, int64_t K);
// yf: optional FP32 carry [B x N]: the low pass also stores its sums there;
// an escalation given it reads only the lo plane and adds to the carry.
hipError_t launch_gemv_low(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                           const uint16_t* scales, uint16_t* y, float* yf, void* ws, size_t ws_bytes,
                           hipStream_t stream);
hipError_t launch_gemv_escalate(const uint16_t* x, int64_t B, int64_t K, int64_t N,
                                const uint8_t* hi, const uint8_t* lo, const uint16_t* scales,
                                const uint8_t* flags, uint16_t* y, float* yf, void* ws, size_t ws_bytes,
                                hipStream_t stream);
// One launch over many problems (rq_gemv_problem table in device memory,
// tile_start set by rq_gemv_group_plan): phase 1 low pass, 2 escalation,
// 3 both.
hipError_t launch_gemv_grouped(const ::rq_gemv_problem* probs, int count, int64_t total_tiles, int64_t B,
                               const uint8_t* flags, int phase, hipStream_t stream);
size_t gate_workspace_bytes(int64_t B, int64_t V);
// The calling thread's current device's copy of the gate scratch (a static
// device array, looked up once per device): its address and size.
hipError_t gate_scratch(void** ptr, size_t* bytes);
hipError_t launch_gate(const uint16_t* logits, int64_t B, int64_t V, float tau, float delta,
                       uint8_t* flags, float* stats, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_kv_quant(const uint16_t* x, int64_t T, int64_t H, int64_t D, uint8_t* codes,
                           float* scales, hipStream_t stream);

}  // namespace rq
