// Dynamic per-32 block quantization of BF16 rows to MXFP4 / MXFP8 with E8M0
// scales, plus the ARCQuant appended columns (residual or copy) and the
// per-channel amax used to pick them.
//
// Steps (Day 0 LLM Inference Support, section V per-group listing; section
// III.3.2 power-of-two scales): group amax -> E8M0 exponent (smallest e
// with amax <= Qmax 2^e) -> round x 2^-e to the element grid.  ARC appends
// follow the ARCQuant page ("Methodologie": residual of the primary stage
// on the selected channels, re-quantized and concatenated along K).
//
// Layout of work: a wave owns 64 consecutive 8-element chunks of one row
// (one 16-byte BF16 load per lane); the four lanes of a quad own one
// 32-element block and share its amax through two DPP quad permutes.  The
// element encode is the hardware scaled conversion (rq_cvt.h), four
// instructions per lane.  Loads and stores of a wave are contiguous (1 KiB
// of BF16 in, 256 B / 512 B of codes out).  HBM-bound.
#include <algorithm>

#include "rq_block.h"
#include "rq_internal.h"

namespace rq {

// Rows are cut into segments of 64 chunks (512 elements), numbered row by
// row; wave w of the grid owns segments w U .. w U + U - 1 and issues all
// their loads before encoding any (U KiB of BF16 in flight per wave).
template <class Fmt, int U>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, uint32_t rows,
                                                         int64_t K, uint32_t segs, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t ldc,
                                                         int64_t lds) {
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  const uint32_t wave = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t cpr = (uint32_t)(K >> 3);  // chunks per row, a multiple of 4
  uint4 q[U];
  uint32_t row[U], c[U];
  bool active[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t unit = wave * (uint32_t)U + (uint32_t)u;
    row[u] = unit / segs;
    c[u] = (unit - row[u] * segs) * 64u + (threadIdx.x & 63u);
    active[u] = row[u] < rows && c[u] < cpr;  // whole quads are in or out
    q[u] = active[u] ? *reinterpret_cast<const uint4*>(x + (int64_t)row[u] * K + (int64_t)c[u] * 8)
                     : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t m = quad_max(amax8(q[u]));
    const uint32_t sb = (uint32_t)(mx_block_exp<Fmt>(m) + 127);
    if (active[u]) {
      encode_store8<Fmt>(q[u], sb, codes + (int64_t)row[u] * ldc + (int64_t)c[u] * 4 * kElemBytesNum);
      if ((c[u] & 3) == 0) scales[(int64_t)row[u] * lds + (c[u] >> 2)] = (uint8_t)sb;
    }
  }
}

// Appended columns: element j of row m comes from channel idx[j]; RESIDUAL
// subtracts the primary stage's dequantized value (exact in fp32: both are
// multiples of the BF16 input's unit in the last place and lie within 2^10
// of each other's scale), COPY takes the channel as is.
template <class Fmt, bool kResidual>
__global__ __launch_bounds__(256) void quant_append_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                           int64_t K, const int32_t* __restrict__ idx,
                                                           int64_t S, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, int64_t ldc,
                                                           int64_t lds) {
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;
  const int64_t cpr = S >> 3;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool active = gid < rows * cpr;
  const int64_t row = active ? gid / cpr : 0;
  const int64_t c = active ? gid - row * cpr : 0;
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t xb = 0;
    if (active) {
      const int32_t ch = idx[c * 8 + i];
      const bool in_range = ch >= 0 && ch < K;  // out-of-range channels read as 0
      xb = in_range ? x[row * K + ch] : 0u;
      if (kResidual && in_range) {
        const int ep = (int)scales[row * lds + (ch >> 5)] - 127;
        const uint32_t code = mx_encode<Fmt>(xb, ep);
        const uint32_t mag = code & ((1u << Fmt::kSignShift) - 1u);
        float dq = __builtin_ldexpf(mx_mag_value<Fmt>(mag), ep);
        if (code >> Fmt::kSignShift) dq = -dq;
        const float r = bf16_to_f32(xb) - dq;
        xb = __builtin_bit_cast(uint32_t, r) >> 16;  // exact: r is a BF16 value
      }
    }
    v[i] = xb;
  }
  const uint4 q = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  const uint32_t m = quad_max(amax8(q));
  const uint32_t sb = (uint32_t)(mx_block_exp<Fmt>(m) + 127);
  if (!active) return;
  encode_store8<Fmt>(q, sb, codes + row * ldc + (K + c * 8) / 2 * kElemBytesNum);
  if ((c & 3) == 0) scales[row * lds + (K >> 5) + (c >> 2)] = (uint8_t)sb;
}

// Primary quantization plus the appended columns in one pass over each row
// (the gather form of the ARC activations and weights: primary blocks in
// the original channel order, appended block j / 32 from channel idx[j]).
// A workgroup owns R consecutive rows and loads all of them before it
// encodes any (thread t holds chunks c = t + 256 i, i < CPT, of each row),
// together with the channel numbers of its appended tasks.  It encodes
// every primary block from registers, as quant_rows_kernel does, and parks
// the row's values in LDS, one buffer per row, with (RESIDUAL) the row's
// block scale bytes.  After the one barrier, task k < R S / 8 (appended
// chunk k mod S / 8 of row k div S / 8, taken by thread k mod 256) gathers
// its eight channels from LDS and encodes them: COPY the values, RESIDUAL
// each value's residual against its primary code (residual1 under its
// block's scale byte), so residuals are formed for the S selected channels
// only.  idx entries outside [0, K) read as 0.
template <class Fmt, bool kResidual, int CPT, int R>
__global__ __launch_bounds__(256) void quant_rows_append_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t K, const int32_t* __restrict__ idx,
                                                                int64_t S, uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  // R rows of K / 8 chunks of BF16 values, then (RESIDUAL) R rows of K / 32
  // block scale bytes
  extern __shared__ uint4 row_lds[];
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  constexpr int kTasks = R;  // appended tasks per thread: R S / 8 <= 256 R
  const int chunks = (int)(K >> 3), s_chunks = (int)(S >> 3), blocks = (int)(K >> 5);
  uint8_t* sb_lds = reinterpret_cast<uint8_t*>(row_lds + R * chunks);
  const int64_t ldc = (K + S) / 2 * kElemBytesNum, lds = (K + S) >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const uint16_t* rh = reinterpret_cast<const uint16_t*>(row_lds);
  const int t = (int)threadIdx.x;
  uint4 q[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = r0 + r < rows;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (r0 + r) * K);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + 256 * i;
      q[r][i] = live && c < chunks ? xr[c] : make_uint4(0, 0, 0, 0);
    }
  }
  int32_t ch[kTasks][8];
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int task = t + 256 * k, c = task % max(s_chunks, 1);
    const bool on = task < R * s_chunks;
#pragma unroll
    for (int e = 0; e < 8; ++e) ch[k][e] = on ? idx[8 * c + e] : -1;
  }
  // chunks is a multiple of 4, so the four lanes of a quad (one 32-block)
  // take the same branches
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = r0 + r;
    if (row >= rows) break;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + 256 * i;
      if (c >= chunks) break;
      const uint32_t sb = (uint32_t)(mx_block_exp<Fmt>(quad_max(amax8(q[r][i]))) + 127);
      const uint2 cv = encode8<Fmt>(q[r][i], sb);
      store8<Fmt>(cv, codes + row * ldc + (int64_t)c * 4 * kElemBytesNum);
      if ((c & 3) == 0) {
        scales[row * lds + (c >> 2)] = (uint8_t)sb;
        if constexpr (kResidual) sb_lds[r * blocks + (c >> 2)] = (uint8_t)sb;
      }
      row_lds[r * chunks + c] = q[r][i];
    }
  }
  __syncthreads();  // every parked row is complete
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int task = t + 256 * k;
    if (task >= R * s_chunks) break;
    const int r = task / s_chunks, c = task - r * s_chunks;
    const int64_t row = r0 + r;
    // whole quads: s_chunks is a multiple of 4, so a quad's four tasks
    // share the row
    if (row < rows) {
      const uint16_t* src = rh + (int64_t)r * K;
      const uint8_t* sbr = sb_lds + r * blocks;
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = ch[k][e] >= 0 && ch[k][e] < K;
        v[e] = in ? (uint32_t)src[ch[k][e]] : 0u;
        if constexpr (kResidual) v[e] = in ? residual1<Fmt>(v[e], sbr[ch[k][e] >> 5]) : 0u;
      }
      const uint4 q2 = pack8(v);
      const uint32_t sb2 = (uint32_t)(mx_block_exp<Fmt>(quad_max(amax8(q2))) + 127);
      encode_store8<Fmt>(q2, sb2, codes + row * ldc + (K + (int64_t)c * 8) / 2 * kElemBytesNum);
      if ((c & 3) == 0) scales[row * lds + (K >> 5) + (c >> 2)] = (uint8_t)sb2;
    }
  }
}

// ARCQuant fused front end (ARCQuant page, technical summary, "Kernel
// Implementatie" with the stages of "Methodologie").  A workgroup owns R
// consecutive rows and loads all of them, and its threads' perm entries,
// before it computes anything; thread t owns chunks c = t + 256 i
// (i < CPT) of every row.  The rows are staged in LDS, one buffer per row;
// with kNorm each row's mean square is summed in fp32 in the order of
// rmsnorm_kernel (lanes by butterfly, then waves 0..3), and every element
// is scaled by 1 / sqrt(ms + eps) and rounded to BF16 as it is gathered, so
// the normalized values equal rmsnorm_kernel's.  One barrier separates the
// staging from the gathers.  Output position j takes channel perm[j]
// (out-of-range entries read as 0).  Primary blocks cover positions
// 0..K-1; the first S positions (the outlier channels after an amax
// reorder) also fill appended block j / 32 + K / 32: the residual against
// the primary stage (kResidual, residual8) or the value itself.
template <class Fmt, bool kResidual, bool kNorm, int CPT, int R>
__global__ __launch_bounds__(256) void arc_frontend_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                                           const int32_t* __restrict__ perm, int64_t S, float eps,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  extern __shared__ uint4 row_lds[];  // R rows of K / 8 chunks of BF16
  __shared__ float sh[R][4];
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  const int chunks = (int)(K >> 3), s_chunks = (int)(S >> 3);
  const int64_t ldc = (K + S) / 2 * kElemBytesNum, lds = (K + S) >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int t = (int)threadIdx.x;
  uint4 q[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = r0 + r < rows;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (r0 + r) * K);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + 256 * i;
      q[r][i] = live && c < chunks ? xr[c] : make_uint4(0, 0, 0, 0);
    }
  }
  int32_t p[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + 256 * i;
    int4 p0 = make_int4(-1, -1, -1, -1), p1 = p0;
    if (c < chunks) {
      p0 = reinterpret_cast<const int4*>(perm)[2 * c];
      p1 = reinterpret_cast<const int4*>(perm)[2 * c + 1];
    }
    p[i][0] = p0.x, p[i][1] = p0.y, p[i][2] = p0.z, p[i][3] = p0.w;
    p[i][4] = p1.x, p[i][5] = p1.y, p[i][6] = p1.z, p[i][7] = p1.w;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + 256 * i;
      if (c >= chunks) break;
      row_lds[r * chunks + c] = q[r][i];
      if constexpr (kNorm) {
        const uint32_t w[4] = {q[r][i].x, q[r][i].y, q[r][i].z, q[r][i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_to_f32(w[e] & 0xFFFFu), b = bf16_to_f32(w[e] >> 16);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
    }
    if constexpr (kNorm) {
      ss = wave_sum(ss);
      if ((t & 63) == 0) sh[r][t >> 6] = ss;
    }
  }
  __syncthreads();  // the staged rows and their partial sums are published
  // chunks and s_chunks are multiples of 4, so the four lanes of a quad
  // (one 32-block) take the same branches
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = r0 + r;
    if (row >= rows) break;
    const uint16_t* rh = reinterpret_cast<const uint16_t*>(row_lds) + (int64_t)r * K;
    float inv = 1.0f;
    if constexpr (kNorm) inv = 1.0f / sqrtf((((sh[r][0] + sh[r][1]) + sh[r][2]) + sh[r][3]) / (float)K + eps);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + 256 * i;
      if (c >= chunks) break;
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (p[i][e] >= 0 && p[i][e] < K) ? (uint32_t)rh[p[i][e]] : 0u;
      uint4 qv;
      if constexpr (kNorm)
        qv = make_uint4(pack_bf16(bf16_to_f32(v[0]) * inv, bf16_to_f32(v[1]) * inv),
                        pack_bf16(bf16_to_f32(v[2]) * inv, bf16_to_f32(v[3]) * inv),
                        pack_bf16(bf16_to_f32(v[4]) * inv, bf16_to_f32(v[5]) * inv),
                        pack_bf16(bf16_to_f32(v[6]) * inv, bf16_to_f32(v[7]) * inv));
      else
        qv = pack8(v);
      const uint32_t sb = (uint32_t)(mx_block_exp<Fmt>(quad_max(amax8(qv))) + 127);
      const uint2 cv = encode8<Fmt>(qv, sb);
      store8<Fmt>(cv, codes + row * ldc + (int64_t)c * 4 * kElemBytesNum);
      if ((c & 3) == 0) scales[row * lds + (c >> 2)] = (uint8_t)sb;
      if (c < s_chunks) {
        const uint4 q2 = kResidual ? residual8<Fmt>(qv, cv, sb) : qv;
        const uint32_t sb2 = (uint32_t)(mx_block_exp<Fmt>(quad_max(amax8(q2))) + 127);
        encode_store8<Fmt>(q2, sb2, codes + row * ldc + (K + (int64_t)c * 8) / 2 * kElemBytesNum);
        if ((c & 3) == 0) scales[row * lds + (K >> 5) + (c >> 2)] = (uint8_t)sb2;
      }
    }
  }
}

// Column amax: a workgroup owns 64 channels; its four waves stride over the
// rows (a wave reads 128 contiguous bytes per row), then combine in LDS.
__global__ __launch_bounds__(256) void channel_amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                           int64_t K, uint16_t* __restrict__ amax) {
  __shared__ uint32_t part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 64 + lane;
  uint32_t m = 0;
  if (col < K)
    for (int64_t r = wave; r < rows; r += 4) m = max(m, (uint32_t)(x[r * K + col] & 0x7FFFu));
  part[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && col < K)
    amax[col] = (uint16_t)max(max(part[0][lane], part[1][lane]), max(part[2][lane], part[3][lane]));
}

static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

template <int U>
static hipError_t launch_quant_rows_u(int fmt, const uint16_t* x, int64_t rows, int64_t K, int64_t segs,
                                      int64_t units, uint8_t* codes, uint8_t* scales, int64_t ldc, int64_t lds,
                                      hipStream_t stream) {
  const unsigned g = (unsigned)((units + 4 * U - 1) / (4 * U));
  if (fmt == 1)
    quant_rows_kernel<FmtE2M1, U><<<g, 256, 0, stream>>>(x, (uint32_t)rows, K, (uint32_t)segs, codes, scales, ldc, lds);
  else
    quant_rows_kernel<FmtE4M3, U><<<g, 256, 0, stream>>>(x, (uint32_t)rows, K, (uint32_t)segs, codes, scales, ldc, lds);
  return hipGetLastError();
}

hipError_t launch_quant_rows(int fmt, const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                             uint8_t* scales, int64_t ldc, int64_t lds, hipStream_t stream) {
  if (rows == 0 || K == 0) return hipSuccess;
  const int64_t segs = (K / 8 + 63) / 64, units = rows * segs;
  if (units > 0x7FFFFFFFll || rows > 0xFFFFFFFFll) return hipErrorInvalidValue;
  // segments per wave: 2 up to 4096 x 3072 (1, 2, 4 and 8 measured on
  // 4096 x 1024 .. 3072), 4 from 32768 segments on (4096 x 4096 MXFP4:
  // 8.0 -> 7.1 us; 8 gave 7.9 us)
  if (units >= 32768) return launch_quant_rows_u<4>(fmt, x, rows, K, segs, units, codes, scales, ldc, lds, stream);
  return launch_quant_rows_u<2>(fmt, x, rows, K, segs, units, codes, scales, ldc, lds, stream);
}

hipError_t launch_quant_append(int fmt, int mode, const uint16_t* x, int64_t rows, int64_t K,
                               const int32_t* idx, int64_t S, uint8_t* codes, uint8_t* scales,
                               int64_t ldc, int64_t lds, hipStream_t stream) {
  const unsigned g = grid_for(rows * (S / 8));
  if (g == 0) return hipSuccess;
  if (fmt == 1) {
    if (mode == 1)
      quant_append_kernel<FmtE2M1, true><<<g, 256, 0, stream>>>(x, rows, K, idx, S, codes, scales, ldc, lds);
    else
      quant_append_kernel<FmtE2M1, false><<<g, 256, 0, stream>>>(x, rows, K, idx, S, codes, scales, ldc, lds);
  } else {
    if (mode == 1)
      quant_append_kernel<FmtE4M3, true><<<g, 256, 0, stream>>>(x, rows, K, idx, S, codes, scales, ldc, lds);
    else
      quant_append_kernel<FmtE4M3, false><<<g, 256, 0, stream>>>(x, rows, K, idx, S, codes, scales, ldc, lds);
  }
  return hipGetLastError();
}

template <class Fmt, int CPT, int R>
static hipError_t launch_rows_append_c(int mode, const uint16_t* x, int64_t rows, int64_t K, const int32_t* idx,
                                       int64_t S, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const size_t shm = (size_t)R * K * 2 + (mode == 1 ? (size_t)R * (K / 32) : 0);
  const unsigned g = (unsigned)((rows + R - 1) / R);
  if (mode == 1)
    quant_rows_append_kernel<Fmt, true, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, idx, S, codes, scales);
  else
    quant_rows_append_kernel<Fmt, false, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, idx, S, codes, scales);
  return hipGetLastError();
}

// Two rows per workgroup up to K = 8192 (16 KiB of LDS at K = 4096: eight
// workgroups per CU), one beyond.
template <class Fmt>
static hipError_t launch_rows_append_f(int mode, const uint16_t* x, int64_t rows, int64_t K, const int32_t* idx,
                                       int64_t S, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (K <= 2048) return launch_rows_append_c<Fmt, 1, 2>(mode, x, rows, K, idx, S, codes, scales, stream);
  if (K <= 4096) return launch_rows_append_c<Fmt, 2, 2>(mode, x, rows, K, idx, S, codes, scales, stream);
  if (K <= 8192) return launch_rows_append_c<Fmt, 4, 2>(mode, x, rows, K, idx, S, codes, scales, stream);
  return launch_rows_append_c<Fmt, 8, 1>(mode, x, rows, K, idx, S, codes, scales, stream);
}

hipError_t launch_quant_rows_append(int fmt, int mode, const uint16_t* x, int64_t rows, int64_t K,
                                    const int32_t* idx, int64_t S, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  const int64_t ldc = fmt == 1 ? (K + S) / 2 : K + S, lds = (K + S) / 32;
  if (rows == 0) return hipSuccess;
  if (S == 0) return launch_quant_rows(fmt, x, rows, K, codes, scales, ldc, lds, stream);
  if (S > 2048 || K > 16384) {
    // beyond one appended chunk per thread or a row in LDS: two passes
    hipError_t e = launch_quant_rows(fmt, x, rows, K, codes, scales, ldc, lds, stream);
    if (e == hipSuccess) e = launch_quant_append(fmt, mode, x, rows, K, idx, S, codes, scales, ldc, lds, stream);
    return e;
  }
  if (fmt == 1) return launch_rows_append_f<FmtE2M1>(mode, x, rows, K, idx, S, codes, scales, stream);
  return launch_rows_append_f<FmtE4M3>(mode, x, rows, K, idx, S, codes, scales, stream);
}

template <class Fmt, int CPT, int R>
static hipError_t launch_frontend_c(int mode, bool norm, const uint16_t* x, int64_t rows, int64_t K,
                                    const int32_t* perm, int64_t S, float eps, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  const size_t shm = (size_t)R * K * 2;
  const unsigned g = (unsigned)((rows + R - 1) / R);
  if (mode == 1 && norm)
    arc_frontend_kernel<Fmt, true, true, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else if (mode == 1)
    arc_frontend_kernel<Fmt, true, false, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else if (norm)
    arc_frontend_kernel<Fmt, false, true, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else
    arc_frontend_kernel<Fmt, false, false, CPT, R><<<g, 256, shm, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  return hipGetLastError();
}

template <class Fmt>
static hipError_t launch_frontend_f(int mode, bool norm, const uint16_t* x, int64_t rows, int64_t K,
                                    const int32_t* perm, int64_t S, float eps, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  // chunks per thread: K / 8 chunks over 256 threads; two rows per
  // workgroup up to K = 8192, one beyond
  if (K <= 2048) return launch_frontend_c<Fmt, 1, 2>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
  if (K <= 4096) return launch_frontend_c<Fmt, 2, 2>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
  if (K <= 8192) return launch_frontend_c<Fmt, 4, 2>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
  return launch_frontend_c<Fmt, 8, 1>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
}

hipError_t launch_arc_frontend(int fmt, int mode, bool norm, const uint16_t* x, int64_t rows, int64_t K,
                               const int32_t* perm, int64_t S, float eps, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (fmt == 1) return launch_frontend_f<FmtE2M1>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
  return launch_frontend_f<FmtE4M3>(mode, norm, x, rows, K, perm, S, eps, codes, scales, stream);
}

hipError_t launch_channel_amax(const uint16_t* x, int64_t rows, int64_t K, uint16_t* amax,
                               hipStream_t stream) {
  const unsigned g = (unsigned)((K + 63) / 64);
  channel_amax_kernel<<<g, 256, 0, stream>>>(x, rows, K, amax);
  return hipGetLastError();
}

}  // namespace rq
