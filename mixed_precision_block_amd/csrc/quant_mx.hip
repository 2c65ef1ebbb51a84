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
  // R row buffers of kRowChunks chunks (the row's K / 8 chunks of BF16
  // values, then a chunk of zeros at kZero that out-of-range idx entries
  // read), then (RESIDUAL) R rows of K / 32 block scale bytes
  extern __shared__ uint4 row_lds[];
  constexpr int kRowChunks = 256 * CPT + 1;
  constexpr uint32_t kZero = 256u * CPT * 16u;
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  constexpr int kTasks = R;  // appended tasks per thread: R S / 8 <= 256 R
  const int chunks = (int)(K >> 3), s_chunks = (int)(S >> 3), blocks = (int)(K >> 5);
  uint8_t* sb_lds = reinterpret_cast<uint8_t*>(row_lds + R * kRowChunks);
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
  // per appended element: LDS byte offset in a row buffer (kZero out of
  // range) and the index of its primary block
  uint32_t off[kTasks][8], blk[kTasks][8];
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int task = t + 256 * k, c = task % max(s_chunks, 1);
    const bool on = task < R * s_chunks;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t chn = on ? (uint32_t)idx[8 * c + e] : 0xFFFFFFFFu;
      const bool in = chn < (uint32_t)K;
      off[k][e] = in ? 2u * chn : kZero;
      blk[k][e] = in ? chn >> 5 : 0u;
    }
  }
  if (t < R) row_lds[t * kRowChunks + 256 * CPT] = make_uint4(0, 0, 0, 0);
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
      row_lds[r * kRowChunks + c] = q[r][i];
    }
  }
  __syncthreads();  // every parked row and its zero chunk is complete
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int task = t + 256 * k;
    if (task >= R * s_chunks) break;
    const int r = task / s_chunks, c = task - r * s_chunks;
    const int64_t row = r0 + r;
    // whole quads: s_chunks is a multiple of 4, so a quad's four tasks
    // share the row
    if (row < rows) {
      const char* rb = reinterpret_cast<const char*>(row_lds + r * kRowChunks);
      const uint8_t* sbr = sb_lds + r * blocks;
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = *reinterpret_cast<const uint16_t*>(rb + off[k][e]);
        if constexpr (kResidual) v[e] = residual1<Fmt>(v[e], sbr[blk[k][e]]);  // 0 stays 0
      }
      const uint4 q2 = pack8(v);
      const uint32_t sb2 = (uint32_t)(mx_block_exp<Fmt>(quad_max(amax8(q2))) + 127);
      encode_store8<Fmt>(q2, sb2, codes + row * ldc + (K + (int64_t)c * 8) / 2 * kElemBytesNum);
      if ((c & 3) == 0) scales[row * lds + (K >> 5) + (c >> 2)] = (uint8_t)sb2;
    }
  }
}

// ARCQuant fused front end (ARCQuant page, technical summary, "Kernel
// Implementatie" with the stages of "Methodologie").  Thread t owns chunks
// c = t + 256 i (i < CPT) of every row.  A row is staged in an LDS row
// buffer of kRowChunks chunks: its K / 8 chunks of BF16, zeros up to chunk
// 256 CPT, then a chunk of zeros at kZero; out-of-range order entries
// point at zeros (the order is turned into LDS addresses once per
// workgroup, so every gather is an unconditional LDS read).  With kNorm the row's mean square is summed in
// fp32 while it is staged, in the order of rmsnorm_kernel (lanes by
// butterfly, then waves 0..3), and every element is scaled by
// 1 / sqrt(ms + eps) and rounded to BF16 as it is gathered, so the
// normalized values equal rmsnorm_kernel's.  Output position j takes
// channel perm[j] (out-of-range entries read as 0).  Primary blocks cover
// positions 0..K-1; the first S positions (the outlier channels after an
// amax reorder) also fill appended block j / 32 + K / 32: the residual
// against the primary stage (kResidual, residual8) or the value itself.
template <int CPT>
struct FeRow {
  static constexpr int kRowChunks = 256 * CPT + 1;
  static constexpr uint32_t kZero = 256u * CPT * 16u;
};

template <int CPT>
__device__ __forceinline__ void fe_load(const uint16_t* __restrict__ x, int64_t row, int64_t K, bool live,
                                        uint4 (&q)[CPT]) {
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
  const int chunks = (int)(K >> 3);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    q[i] = live && c < chunks ? xr[c] : make_uint4(0, 0, 0, 0);
  }
}

typedef __attribute__((address_space(3))) uint4 lds_uint4;
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;

// LDS address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
  return (uint32_t)(uintptr_t)(const lds_uint4*)p;
}

// LDS addresses, in the row buffer at LDS address base, of the channels
// this thread's chunks gather
template <int CPT>
__device__ __forceinline__ void fe_offsets(const int32_t* __restrict__ perm, int64_t K, uint32_t base,
                                           uint32_t (&po)[CPT][8]) {
  const int chunks = (int)(K >> 3);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    int4 p0 = make_int4(-1, -1, -1, -1), p1 = p0;
    if (c < chunks) {
      p0 = reinterpret_cast<const int4*>(perm)[2 * c];
      p1 = reinterpret_cast<const int4*>(perm)[2 * c + 1];
    }
    const int32_t pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    // entries in [K, 2048 CPT) read the buffer's zero tail, larger and
    // negative ones (as unsigned) the zero chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) po[i][e] = base + 2u * min((uint32_t)pv[e], FeRow<CPT>::kZero / 2u);
  }
}

// Stage one row in buf, its chunks past K / 8 as zeros (fe_load leaves
// them zero); with kNorm, sh_row[w] = wave w's sum of squares (the zeros
// add nothing).
template <bool kNorm, int CPT>
__device__ __forceinline__ void fe_stage(const uint4 (&q)[CPT], uint4* buf, float* sh_row) {
  const int t = (int)threadIdx.x;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + 256 * i;
    buf[c] = q[i];
    if constexpr (kNorm) {
      const uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
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
    if ((t & 63) == 0) sh_row[t >> 6] = ss;
  }
}

// Gather, normalize, quantize and store one staged row.
// (po holds LDS addresses in the first row buffer; this row's buffer lies
// buf_off bytes further)
// The normalization factor of a row from its four wave sums, as
// rmsnorm_kernel forms it.
__device__ __forceinline__ float fe_inv(const float* sh_row, int64_t K, float eps) {
  return 1.0f / sqrtf((((sh_row[0] + sh_row[1]) + sh_row[2]) + sh_row[3]) / (float)K + eps);
}

// (inv: the row's normalization factor, used with kNorm)
template <class Fmt, bool kResidual, bool kNorm, int CPT>
__device__ __forceinline__ void fe_emit(uint32_t buf_off, float inv, const uint32_t (&po)[CPT][8], int64_t row,
                                        int64_t K, int64_t S, uint8_t* __restrict__ codes,
                                        uint8_t* __restrict__ scales) {
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  const int chunks = (int)(K >> 3), s_chunks = (int)(S >> 3);
  const int64_t ldc = (K + S) / 2 * kElemBytesNum, lds = (K + S) >> 5;
  // chunks and s_chunks are multiples of 4, so the four lanes of a quad
  // (one 32-block) take the same branches
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    if (c >= chunks) break;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *(lds_cu16*)(uintptr_t)(po[i][e] + buf_off);
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

// A workgroup owns R consecutive rows and loads all of them, and its
// order offsets, before it computes anything; one barrier separates the
// staging of the R rows (a buffer each) from their gathers (with kNorm a
// second one publishes each row's factor, formed once by wave r).
template <class Fmt, bool kResidual, bool kNorm, int CPT, int R>
__global__ __launch_bounds__(256) void arc_frontend_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                                           const int32_t* __restrict__ perm, int64_t S, float eps,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  // R row buffers (static, so their LDS address is known when the kernel
  // is compiled and the gathers' addresses need no add), the R rows' four
  // wave sums
  constexpr int kRowChunks = FeRow<CPT>::kRowChunks;
  __shared__ uint4 row_lds[R * kRowChunks];
  __shared__ float sh[R][4];
  __shared__ float sh_inv[R];
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int t = (int)threadIdx.x;
  uint4 q[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) fe_load<CPT>(x, r0 + r, K, r0 + r < rows, q[r]);
  uint32_t po[CPT][8];
  fe_offsets<CPT>(perm, K, lds_addr(row_lds), po);
  if (t < R) row_lds[t * kRowChunks + 256 * CPT] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < R; ++r) fe_stage<kNorm, CPT>(q[r], row_lds + r * kRowChunks, sh[r]);
  __syncthreads();  // the staged rows, their zero chunks and partial sums are published
  if constexpr (kNorm) {
    // wave r forms row r's factor once for the workgroup (R <= 4 waves)
    const int w = t >> 6;
    if (w < R && (t & 63) == 0) sh_inv[w] = fe_inv(sh[w], K, eps);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r0 + r >= rows) break;
    fe_emit<Fmt, kResidual, kNorm, CPT>(16u * r * kRowChunks, kNorm ? sh_inv[r] : 1.0f, po, r0 + r, K, S, codes,
                                        scales);
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
  const size_t shm = (size_t)R * (256 * CPT + 1) * 16 + (mode == 1 ? (size_t)R * (K / 32) : 0);
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
  const unsigned g = (unsigned)((rows + R - 1) / R);
  if (mode == 1 && norm)
    arc_frontend_kernel<Fmt, true, true, CPT, R><<<g, 256, 0, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else if (mode == 1)
    arc_frontend_kernel<Fmt, true, false, CPT, R><<<g, 256, 0, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else if (norm)
    arc_frontend_kernel<Fmt, false, true, CPT, R><<<g, 256, 0, stream>>>(x, rows, K, perm, S, eps, codes, scales);
  else
    arc_frontend_kernel<Fmt, false, false, CPT, R><<<g, 256, 0, stream>>>(x, rows, K, perm, S, eps, codes, scales);
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
