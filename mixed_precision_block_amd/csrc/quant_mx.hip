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
// Layout of work: one thread owns 8 consecutive elements (one 16-byte BF16
// load); the four threads of a lane quad own one 32-element block and share
// its amax through two DPP quad permutes.  Loads and stores of a wave are
// contiguous (1 KiB of BF16 in, 256 B / 512 B of codes out).  HBM-bound.
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
  return m;
}

// Encode 8 BF16 values (bit patterns in v[0..7]) with block exponent e and
// store them: FP4 -> one dword (element 2j in the low nibble of byte j),
// FP8 -> two dwords.
template <class Fmt>
__device__ __forceinline__ void encode_store8(const uint32_t v[8], int e, uint8_t* dst) {
  if constexpr (Fmt::kMantBits == 1) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= mx_encode<Fmt>(v[i], e) << (4 * i);
    *reinterpret_cast<uint32_t*>(dst) = w;
  } else {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= mx_encode<Fmt>(v[i], e) << (8 * i);
      w1 |= mx_encode<Fmt>(v[4 + i], e) << (8 * i);
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
  }
}

template <class Fmt>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                         int64_t K, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t ldc,
                                                         int64_t lds) {
  constexpr int kElemBytesNum = Fmt::kMantBits == 1 ? 1 : 2;  // bytes per 2 elements
  const int64_t cpr = K >> 3;  // 8-element chunks per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool active = gid < rows * cpr;  // whole quads are in or out (cpr % 4 == 0)
  const int64_t row = active ? gid / cpr : 0;
  const int64_t c = active ? gid - row * cpr : 0;
  uint4 q = make_uint4(0, 0, 0, 0);
  if (active) q = *reinterpret_cast<const uint4*>(x + row * K + c * 8);
  uint32_t v[8] = {q.x & 0xFFFFu, q.x >> 16, q.y & 0xFFFFu, q.y >> 16,
                   q.z & 0xFFFFu, q.z >> 16, q.w & 0xFFFFu, q.w >> 16};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, v[i] & 0x7FFFu);
  m = quad_max(m);
  const int e = mx_block_exp<Fmt>(m);
  if (!active) return;
  encode_store8<Fmt>(v, e, codes + row * ldc + c * 4 * kElemBytesNum);
  if ((c & 3) == 0) scales[row * lds + (c >> 2)] = (uint8_t)(e + 127);
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
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, v[i] & 0x7FFFu);
  m = quad_max(m);
  const int e = mx_block_exp<Fmt>(m);
  if (!active) return;
  encode_store8<Fmt>(v, e, codes + row * ldc + (K + c * 8) / 2 * kElemBytesNum);
  if ((c & 3) == 0) scales[row * lds + (K >> 5) + (c >> 2)] = (uint8_t)(e + 127);
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

hipError_t launch_quant_rows(int fmt, const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                             uint8_t* scales, int64_t ldc, int64_t lds, hipStream_t stream) {
  const unsigned g = grid_for(rows * (K / 8));
  if (g == 0) return hipSuccess;
  if (fmt == 1)
    quant_rows_kernel<FmtE2M1><<<g, 256, 0, stream>>>(x, rows, K, codes, scales, ldc, lds);
  else
    quant_rows_kernel<FmtE4M3><<<g, 256, 0, stream>>>(x, rows, K, codes, scales, ldc, lds);
  return hipGetLastError();
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

hipError_t launch_channel_amax(const uint16_t* x, int64_t rows, int64_t K, uint16_t* amax,
                               hipStream_t stream) {
  const unsigned g = (unsigned)((K + 63) / 64);
  channel_amax_kernel<<<g, 256, 0, stream>>>(x, rows, K, amax);
  return hipGetLastError();
}

}  // namespace rq
