/*
 * rq.h -- C ABI of librq: block-quantized matrix multiplication with a
 * selective high-precision path, native to AMD Instinct MI355X (gfx950).
 *
 * Every tensor argument is a plain pointer; unless stated otherwise it is a
 * DEVICE pointer to memory the caller allocated and owns.  `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).  All compute calls
 * are asynchronous on that stream: they validate their arguments on the
 * host, enqueue kernels and return.  On a validation error nothing is
 * enqueued.  Device faults surface at the caller's next synchronization.
 * A tensor with no elements (one of its extents is 0) is never read or
 * written, and its pointer may be NULL; a call whose work is empty
 * validates its other arguments and enqueues nothing.
 * No call allocates device memory; calls that need scratch space take a
 * caller-provided workspace whose size a *_workspace_bytes() helper gives.
 * The library keeps no per-call state and is thread-safe (the last-error
 * string is thread-local).
 *
 * Layouts (all row-major, "K-major" = the reduction dimension contiguous):
 *   BF16 tensors       uint16 bit patterns.
 *   MXFP4 codes        E2M1, two per byte along K: element 2j in bits 3:0,
 *                      element 2j+1 in bits 7:4; a row of K elements takes
 *                      K/2 bytes.
 *   MXFP8 codes        E4M3FN, one byte per element.
 *   MX scales          E8M0, one byte per (row, 32-element block along K),
 *                      [rows x K/32]; byte b means 2^(b-127).
 *
 * Inputs must be finite; behaviour on Inf/NaN inputs is unspecified.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_ABI_VERSION 5

typedef enum {
  RQ_OK = 0,
  RQ_EINVAL = 1, /* null pointer, unknown enum, inconsistent idx/S/append   */
  RQ_ESHAPE = 2, /* K or S not a multiple of 32, B outside [1,16], steps
                    outside [1,64], workspace too small, negative size      */
  RQ_EALIGN = 3, /* a pointer is not 16-byte aligned                         */
  RQ_EHIP = 4,   /* a HIP runtime call failed; detail in rq_last_error()     */
  RQ_ENODEV = 5  /* no HIP device is visible                                 */
} rq_status;

/* element formats (RQ_MXFP8_F8MFMA: rq_gemm only, on RQ_MXFP8 codes) */
enum { RQ_MXFP4 = 1, RQ_MXFP8 = 2, RQ_BF16 = 3, RQ_MXFP8_F8MFMA = 4 };
/* rq_quantize append modes */
enum { RQ_APPEND_NONE = 0, RQ_APPEND_RESIDUAL = 1, RQ_APPEND_COPY = 2 };
/* GEMM output types */
enum { RQ_OUT_BF16 = 0, RQ_OUT_F32 = 1 };
/* GEMV phases */
enum { RQ_LOW = 1, RQ_ESCALATE = 2, RQ_BOTH = 3 };

int rq_abi_version(void);
const char *rq_status_str(rq_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char *rq_last_error(void);

/*
 * rq_quantize -- dynamic per-32-element block quantization of BF16 rows.
 *
 * Defines: Day 0 LLM Inference Support (Baidu AI Cloud), section V, the
 * per-group quantization listing (group amax, scale from amax and the
 * format maximum with an all-zero group at scale 1, clip, round to
 * nearest-even), with section III.3.2's power-of-two scales: the block
 * exponent is the smallest e with amax <= Qmax * 2^e (Qmax = 6 for E2M1,
 * 448 for E4M3), clamped to [-127, 127]; an all-zero block gets e = 0.
 * Elements are x * 2^-e rounded to nearest, ties to even; a negative value
 * that rounds to zero keeps its sign.
 *
 * ARC appends (ARCQuant: Boosting NVFP4 Quantization with Augmented
 * Residual Channels, technical summary, "Methodologie", dual-stage
 * quantization and augmented GEMM): with S > 0 and idx[S] (device int32,
 * each in [0, K), duplicates allowed; an entry outside [0, K) cannot be
 * checked on the host and reads as channel value 0) the output has
 * K' = K + S columns:
 *   RQ_APPEND_RESIDUAL  columns K+j hold Q(x[:, idx[j]] - deq(Q(x))[:, idx[j]])
 *                       (the exact residual of the primary stage; activations)
 *   RQ_APPEND_COPY      columns K+j hold Q(x[:, idx[j]])  (duplicated weight
 *                       columns, W' = [W | W[:, idx]])
 * Appended columns form their own blocks of 32 consecutive j.
 *
 * x_bf16  [rows x K] BF16, 16-byte aligned.   K % 32 == 0, S % 32 == 0.
 * fmt     RQ_MXFP4 or RQ_MXFP8.
 * codes   [rows x K'] elements (FP4: K'/2 bytes per row), 16-byte aligned.
 * scales  [rows x K'/32] bytes.
 * append  RQ_APPEND_NONE requires idx == NULL and S == 0.
 */
rq_status rq_quantize(const void *x_bf16, int64_t rows, int64_t K, int fmt,
                      const int32_t *idx, int64_t S, int append, void *codes,
                      uint8_t *scales, void *stream);

/*
 * rq_channel_amax -- per-channel absolute maximum over all rows, the
 * ranking statistic of ARCQuant's outlier-channel identification (same
 * page, "Methodologie", adaptive outlier identification).
 * x_bf16 [rows x K] BF16; amax_bf16 [K] BF16 bit patterns (device).
 */
rq_status rq_channel_amax(const void *x_bf16, int64_t rows, int64_t K,
                          uint16_t *amax_bf16, void *stream);

/*
 * rq_select_channels -- HOST helper: the S channels with the largest amax,
 * in descending amax order, ties to the lower channel index.  amax_bf16
 * [K] and idx [S] are HOST pointers.  Synchronous; no device work.
 */
rq_status rq_select_channels(const uint16_t *amax_bf16, int64_t K, int64_t S,
                             int32_t *idx);

/*
 * rq_arc_frontend -- the fused ARC front end: channel reorder, RMSNorm,
 * primary and residual quantization in one pass, producing the augmented
 * row the GEMM consumes (ARCQuant page, technical summary, "Kernel
 * Implementatie", with the stages of "Methodologie").
 *   n = rmsnorm ? bf16(x / sqrt(mean(x^2) + eps)) : x   per row, no gain
 *       (the RMSNorm of the recurrent block, RAMP page section 4.2; fp32
 *       sum of squares, the same values as rq_rmsnorm)
 *   p[j] = n[perm[j]]                    j < K (perm[j] outside [0, K) reads 0)
 *   codes/scales[:, 0:K]   = Q(p)         primary blocks
 *   codes/scales[:, K:K+S] = Q(p[:S] - deq(Q(p))[:S])   RQ_APPEND_RESIDUAL
 *                          = Q(p[:S])                   RQ_APPEND_COPY
 * With perm ordering the channels by descending calibration amax
 * (rq_select_channels with S = K), p[:S] are the S outlier channels, so
 * the residual blocks need no gather.  Activations take
 * RQ_APPEND_RESIDUAL; the weights W' for the same perm take RQ_APPEND_COPY
 * with rmsnorm = 0, and rq_gemm over K + S multiplies them.
 * x_bf16 [rows x K] BF16; perm [K] int32 (device, 16-byte aligned);
 * codes [rows x (K+S)] elements (FP4 packed two per byte), scales
 * [rows x (K+S)/32] E8M0.  fmt RQ_MXFP4 / RQ_MXFP8.  append
 * RQ_APPEND_NONE exactly when S == 0.  rmsnorm 0 or 1, eps finite >= 0.
 * 0 < K <= 16384 (the row is staged in LDS), K % 32 == 0, 0 <= S <= K,
 * S % 32 == 0.  x, perm, codes 16-byte aligned.
 */
rq_status rq_arc_frontend(const void *x_bf16, int64_t rows, int64_t K,
                          const int32_t *perm, int64_t S, int fmt, int append,
                          int rmsnorm, float eps, void *codes, uint8_t *scales,
                          void *stream);

/*
 * rq_rmsnorm -- out = bf16(h / sqrt(mean(h^2) + eps)) per row, no gain: the
 * normalization of the recurrent block (RAMP page, section 4.2; BF16 around
 * the contractions), used inside rq_recurrent_prefill and for calibrating
 * the ARC channel order on normalized activations.  fp32 sum of squares
 * in a fixed order.  h_bf16, out_bf16 [rows x D] BF16, D % 8 == 0, 16-byte
 * aligned; eps finite >= 0.
 */
rq_status rq_rmsnorm(const void *h_bf16, int64_t rows, int64_t D, float eps,
                     void *out_bf16, void *stream);

/*
 * rq_gemm -- Y[M x N] = A . W^T with FP32 accumulation.
 *
 * Defines: the unified block-scaled GEMM of the ARCQuant page (technical
 * summary, "Methodologie": one GEMM whose accumulator adds every K term)
 * and the Day-0 page's section V item 3 (block scales consumed inside the
 * multiply-accumulate):
 *   Y[m,n] = sum_b 2^(ea[m,b] + ew[n,b] - 254) * sum_{k in b} qa[m,k] qw[n,k]
 * fmt     RQ_MXFP4 / RQ_MXFP8: a, w are codes, a_scales [M x K/32] and
 *         w_scales [N x K/32] are E8M0 bytes.  Every product is exact and
 *         the sum is accumulated in FP32 (MXFP4 on the FP4 scaled matrix
 *         instruction, whose products are exact; MXFP8 codes dequantized to
 *         BF16 in registers, exact for block exponents >= -117, and summed
 *         on the BF16 matrix instruction).
 *         RQ_MXFP8_F8MFMA: the RQ_MXFP8 codes and scales on gfx950's FP8
 *         scaled matrix instruction, at twice the BF16 instruction's rate
 *         but NOT an FP32 accumulation of exact products: the instruction
 *         sums each run of 8 consecutive K terms after aligning the products
 *         to the run's largest exponent-field sum E (an E4M3 subnormal
 *         counts as exponent -6) and truncating each toward zero to a
 *         multiple of 2^(E - 13), times the block scales.  The error is at
 *         most 2^-10 sum_k |a_k w_k| per output (about 4e-5 relative
 *         Frobenius on normally distributed operands).
 *         RQ_BF16: a [M x K], w [N x K] are BF16; the scale pointers must be
 *         NULL.
 * out     RQ_OUT_BF16 (round to nearest even) or RQ_OUT_F32; y [M x N].
 * M, N >= 1 arbitrary; K % 32 == 0.  a, w, y 16-byte aligned.
 * Deterministic: no atomics, a fixed accumulation order per element.
 */
rq_status rq_gemm(int fmt, const void *a, const uint8_t *a_scales,
                  const void *w, const uint8_t *w_scales, int64_t M, int64_t N,
                  int64_t K, int out, void *y, void *stream);

/*
 * rq_gemm_arc -- ARCQuant GEMM on MXFP4: quantizes the BF16 activations
 * with RQ_APPEND_RESIDUAL into the workspace (A' = [Q(A) | Q(r)],
 * K' = K + S), then runs rq_gemm(RQ_MXFP4) over K'.
 * w_aug / w_aug_scales: W' from rq_quantize(W, RQ_MXFP4, idx, S,
 * RQ_APPEND_COPY) with the same idx.
 * Defines: ARCQuant page, technical summary, "Methodologie" (augmented
 * matrix multiplication over (N, K_in + S, M)).
 */
size_t rq_gemm_arc_workspace_bytes(int64_t M, int64_t K, int64_t S);
rq_status rq_gemm_arc(const void *a_bf16, int64_t M, int64_t K,
                      const int32_t *idx, int64_t S, const void *w_aug,
                      const uint8_t *w_aug_scales, int64_t N, void *workspace,
                      size_t ws_bytes, int out, void *y, void *stream);

/*
 * rq_recurrent_prefill -- RAMP recurrent-depth prefill of a shared block.
 *
 * Defines: RAMP: Recurrent Adaptive Mixed Precision for Efficient Prefill
 * in Recurrent-Depth Language Models, sections 2.1 (a shared block applied
 * repeatedly), 2.3 (a per-step precision schedule), 4.1 (low precision
 * before the switch, reference precision after) and 4.2 (low-precision
 * weights quantized once, activations quantized dynamically, everything
 * else BF16).  Block, applied `steps` times in place on h:
 *   n = bf16(RMSNorm(h)) (eps, no gain); z = bf16(n W1^T);
 *   u = bf16(SiLU(z)); v = bf16(u W2^T); h = bf16(h + v).
 * Bit t-1 of `schedule` set: step t quantizes n and u with `fmt` and uses
 * the quantized weights w1_q/w1_s, w2_q/w2_s (from rq_quantize); clear:
 * BF16 operands w1_bf16/w2_bf16.  Both weight copies stay resident.
 * fmt: RQ_MXFP4, RQ_MXFP8 (exact block-scaled GEMMs), or RQ_MXFP8_F8MFMA:
 * n and u quantized to MXFP8 as with RQ_MXFP8 (weights from
 * rq_quantize(.., RQ_MXFP8)) and the quantized steps' GEMMs on the FP8
 * scaled instruction, whose products are truncated inside runs of 8 K
 * terms (see rq_gemm).
 * h_bf16 [S x D] in/out; w1 [F x D]; w2 [D x F]; D % 32 == 0, F % 32 == 0.
 * steps in [1, 64].  Quantized weight pointers may be NULL when no
 * schedule bit below `steps` is set; BF16 ones when every bit is set.
 */
size_t rq_recurrent_prefill_workspace_bytes(int64_t S, int64_t D, int64_t F,
                                            int fmt);
rq_status rq_recurrent_prefill(void *h_bf16, int64_t S, int64_t D, int64_t F,
                               const void *w1_bf16, const void *w2_bf16,
                               const void *w1_q, const uint8_t *w1_s,
                               const void *w2_q, const uint8_t *w2_s, int fmt,
                               uint64_t schedule, int steps, float eps,
                               void *workspace, size_t ws_bytes, void *stream);

/*
 * rq_pack_nibble_planes -- offline packing of int8 weights for the decode
 * GEMV (Escalating Weight Precision Only When Decoding Becomes Uncertain,
 * setup paragraph: 8-bit storage read first through the top four bits).
 *   hi = w >> 4 (arithmetic, -8..7, stored as 4-bit two's complement)
 *   lo = w & 15 (0..15)
 * w [N x K] int8, scales_f16 [N x K/32] FP16 (row-major inputs).
 * Outputs use a row-tiled layout made for coalesced GEMV loads; N is
 * padded to Np = ceil(N/64)*64 (padding rows get zero weights and scales):
 *   plane byte of (row n, block b = k/32, byte i in 0..15) at
 *     ((n/64) * (K/32) + b) * 1024 + (n%64) * 16 + i
 *   within a row's 16 bytes, little-endian dword q (0..3) holds element
 *     k = 32b + 8q + 2j in bits 4j+3..4j and k+1 in bits 4j+19..4j+16
 *     (j = 0..3);
 *   scale of (n, b) at ((n/64) * (K/32) + b) * 64 + (n%64).
 * hi, lo: rq_nibble_plane_bytes(N, K) bytes each; scales_tiled:
 * rq_nibble_scale_bytes(N, K) bytes; the planes 16-byte aligned.
 */
size_t rq_nibble_plane_bytes(int64_t N, int64_t K);
size_t rq_nibble_scale_bytes(int64_t N, int64_t K);
rq_status rq_pack_nibble_planes(const int8_t *w, const uint16_t *scales_f16,
                                int64_t N, int64_t K, uint8_t *hi, uint8_t *lo,
                                uint16_t *scales_tiled, void *stream);

/*
 * rq_gemv_nibble_escalate -- decode GEMV with top-nibble low pass and 8-bit
 * recompute of flagged tokens (same article, setup paragraph).
 *   RQ_LOW       y[t,n] = sum_b s[n,b] sum_{k in b} 16*hi[n,k] x[t,k], all t < B
 *   RQ_ESCALATE  rows t with flags[t] != 0 are recomputed with
 *                w = 16*hi + lo and overwritten; exits early when no flag
 *                is set
 *   RQ_BOTH      RQ_LOW then RQ_ESCALATE
 * x_bf16 [B x K] BF16 with B in [1, 16]; planes/scales from
 * rq_pack_nibble_planes; x and planes 16-byte aligned; flags [B] uint8
 * (device; may be NULL for RQ_LOW); y_bf16 [B x N] BF16.  FP32
 * accumulation, BF16 output.
 * workspace: device scratch of ws_bytes >= rq_gemv_workspace_bytes(B, N,
 * K) bytes (caller-owned, 16-byte aligned) lets shapes with few 64-row
 * tiles split K over more workgroups within the one launch: each writes
 * FP32 partial sums and bumps a per-tile arrival counter kept in the
 * workspace's first 32 KiB (one counter per 128-byte line), and the last to
 * arrive adds the partials in a fixed order and resets the counter.  Those
 * 32 KiB must be ZERO before the first call (zero the workspace once after
 * allocating it); every call leaves them zero again, so the workspace can
 * be reused by later calls of
 * any shape and by graph replays.  Calls sharing a workspace must not
 * overlap.
 * NULL / smaller runs the shape unsplit.  The result is the same bits
 * either way only up to FP32 summation order; a given (shape, workspace)
 * choice is deterministic.
 * y_f32: optional FP32 carry [B x N] (caller-owned, 4-byte aligned, NULL
 * for none).  RQ_LOW with it also stores every row's unrounded FP32 sum.
 * RQ_ESCALATE with it takes those sums as the hi part -- they must come
 * from an RQ_LOW on the same x, planes, shape and workspace choice, with
 * this y_f32 -- and reads only the lo plane (half the bytes):
 * y[t,n] = BF16(y_f32[t,n] + sum_b s[n,b] sum_k lo[n,k] x[t,k]), exact
 * in real arithmetic because w = 16*hi + lo; w_hi may then be NULL for
 * RQ_ESCALATE alone.  The flagged rows of y_f32 are left unchanged.
 */
size_t rq_gemv_workspace_bytes(int64_t B, int64_t N, int64_t K);
rq_status rq_gemv_nibble_escalate(const void *x_bf16, int64_t B, int64_t K,
                                  int64_t N, const uint8_t *w_hi,
                                  const uint8_t *w_lo,
                                  const uint16_t *scales_tiled,
                                  const uint8_t *flags, int phase,
                                  void *workspace, size_t ws_bytes,
                                  float *y_f32, void *y_bf16, void *stream);

/*
 * Grouped decode GEMV: one launch over many independent problems (the same
 * operation as rq_gemv_nibble_escalate on each, same B and flags), for
 * decode steps whose linears are launch-latency bound one by one.
 *
 * rq_gemv_problem: one problem; pointers as for rq_gemv_nibble_escalate
 * (every x holds the same B tokens; w_lo may be NULL, and such a problem
 * then takes only the low pass: the escalation skips it; y_f32 is the
 * optional carry, with the same meaning per problem).  tile_start is
 * filled by rq_gemv_group_plan.
 *
 * rq_gemv_group_plan (host): validates every entry (non-NULL x, w_hi,
 * scales_tiled and y; N > 0; K > 0 with K % 32 == 0; 16-byte aligned x and
 * planes), sets tile_start to the running sum of ceil(N / 64), and returns
 * the total number of 64-row tiles, or -1 (with rq_last_error) if an entry
 * is invalid or count < 1.
 *
 * rq_gemv_nibble_escalate_grouped: problems_dev is the planned array
 * copied unchanged to device memory (count entries, 16-byte aligned,
 * caller-owned); total_tiles is the plan's return value (workgroups past
 * the last problem's tiles do nothing).  B in [1, 16]; flags as for
 * rq_gemv_nibble_escalate, shared by all problems.  The device table is
 * not validated again: it must be the plan's output.  Outputs are
 * bit-identical to unsplit rq_gemv_nibble_escalate calls on each problem.
 */
typedef struct rq_gemv_problem {
  const void *x_bf16;           /* [B x K] BF16 */
  const uint8_t *w_hi;          /* hi plane */
  const uint8_t *w_lo;          /* lo plane, or NULL for RQ_LOW only */
  const uint16_t *scales_tiled; /* tiled FP16 scales */
  void *y_bf16;                 /* [B x N] BF16 */
  float *y_f32;                 /* optional FP32 carry [B x N], or NULL */
  int64_t N, K;
  int64_t tile_start;           /* set by rq_gemv_group_plan */
} rq_gemv_problem;

int64_t rq_gemv_group_plan(rq_gemv_problem *problems, int count);
rq_status rq_gemv_nibble_escalate_grouped(const rq_gemv_problem *problems_dev,
                                          int count, int64_t total_tiles,
                                          int64_t B, const uint8_t *flags,
                                          int phase, void *stream);

/*
 * rq_escalation_gate -- entropy / margin gate over low-pass logits (same
 * article, setup paragraph: recompute when the output distribution's
 * entropy is above a threshold or the top-1/top-2 probability gap is
 * small).  flags[t] = (H(softmax(logits[t])) > tau) || (p1 - p2 < delta).
 * logits_bf16 [B x V] (finite, 2-byte aligned); flags [B] uint8; stats [B x 2] float
 * (entropy in nats, p1 - p2; 4-byte aligned) or NULL.  B in [1, 16],
 * 2 <= V < 2^31.  FP32 arithmetic.
 * workspace: device scratch of ws_bytes >= rq_escalation_gate_workspace_bytes
 * (B, V) bytes (caller-owned, 16-byte aligned, contents irrelevant) lets
 * each row split over many workgroups whose partial statistics a second
 * kernel merges; NULL / smaller takes one workgroup per row.  The two
 * differ only in FP32 summation order; each is deterministic.
 */
size_t rq_escalation_gate_workspace_bytes(int64_t B, int64_t V);
rq_status rq_escalation_gate(const void *logits_bf16, int64_t B, int64_t V,
                             float tau, float delta, uint8_t *flags,
                             float *stats, void *workspace, size_t ws_bytes,
                             void *stream);

/*
 * rq_escalation_gate_noalloc -- rq_escalation_gate with the split-row
 * kernels, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as rq_escalation_gate given a workspace of
 * rq_escalation_gate_workspace_bytes(B, V); the per-range statistics go to
 * a static 16 KiB device scratch instead (each GPU the library runs on
 * holds one until the process ends; B <= 16 always fits, a larger need
 * returns RQ_ESHAPE).  It calls no allocating routine: the scratch's
 * device address is looked up once per device, on its first call there.
 * Calls on one GPU share that GPU's scratch, so calls that overlap on one
 * GPU (concurrent streams, threads) race; calls in one stream are ordered.
 * Nothing in the scratch needs clearing: every call overwrites what it
 * reads.
 */
rq_status rq_escalation_gate_noalloc(const void *logits_bf16, int64_t B,
                                     int64_t V, float tau, float delta,
                                     uint8_t *flags, float *stats,
                                     void *stream);

/*
 * rq_kv_quantize -- FP8 per-token-head-tile quantize-on-write (Day 0 LLM
 * Inference Support, section III.3.3, tile = 128, with the section V
 * listing's scale rule): per (token, head, 128-element tile),
 * scale = amax/448 in float32 (1 for an all-zero tile),
 * codes = E4M3FN(clip(x / scale, +-448)) with float32 division.
 * x_bf16 [T x H x D] with D % 128 == 0; codes [T x H x D]; scales
 * [T x H x D/128] float32.
 */
rq_status rq_kv_quantize(const void *x_bf16, int64_t T, int64_t H, int64_t D,
                         uint8_t *codes, float *scales, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RQ_H */
