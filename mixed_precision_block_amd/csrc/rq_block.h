// Device-only helpers shared by the row-wise kernels: quad, wave and
// 256-thread block reductions, and the encode-and-store of eight BF16
// values into one MX block's codes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq_cvt.h"
#include "rq_device.h"

namespace rq {

// Max over the four lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1]);
// all four lanes must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
  return m;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a 256-thread block in a fixed order (lanes by butterfly, then
// waves 0..3).  Every thread gets the sum; contains two block barriers.
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

// Largest BF16 magnitude field of eight values (element 2i in the low half
// of dword i): the fields masked in place, a packed 16-bit unsigned max
// over the dwords, then the larger half.
typedef unsigned short rq_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t amax8(uint4 q) {
  const rq_u16x2 a = __builtin_bit_cast(rq_u16x2, q.x & 0x7FFF7FFFu);
  const rq_u16x2 b = __builtin_bit_cast(rq_u16x2, q.y & 0x7FFF7FFFu);
  const rq_u16x2 c = __builtin_bit_cast(rq_u16x2, q.z & 0x7FFF7FFFu);
  const rq_u16x2 d = __builtin_bit_cast(rq_u16x2, q.w & 0x7FFF7FFFu);
  const rq_u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

__device__ __forceinline__ uint4 pack8(const uint32_t v[8]) {
  return make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
}

// Codes of 8 BF16 values under block scale byte sb: FP4 -> .x (element k
// in nibble k), FP8 -> .x, .y (element k in byte k).
template <class Fmt>
__device__ __forceinline__ uint2 encode8(uint4 q, uint32_t sb) {
  const float scale = e8m0_to_f32(sb);
  if constexpr (Fmt::kMantBits == 1)
    return make_uint2(cvt8_e2m1(q, scale), 0u);
  else
    return cvt8_e4m3(q, scale);
}

// Code of element k of an encode8 result.
template <class Fmt>
__device__ __forceinline__ uint32_t code_at(uint2 c, int k) {
  if constexpr (Fmt::kMantBits == 1)
    return (c.x >> (4 * k)) & 0xFu;
  else
    return ((k < 4 ? c.x : c.y) >> (8 * (k & 3))) & 0xFFu;
}

template <class Fmt>
__device__ __forceinline__ void store8(uint2 c, uint8_t* dst) {
  if constexpr (Fmt::kMantBits == 1)
    *reinterpret_cast<uint32_t*>(dst) = c.x;
  else
    *reinterpret_cast<uint2*>(dst) = c;
}

// Residuals of 8 BF16 values against their codes c under block scale byte
// sb: x - deq(code), as BF16 bit patterns.  The codes are dequantized by
// the hardware scaled conversion to float (exact: a power-of-two scaling
// of a grid value) and the difference is exact in float: both terms are
// multiples of the smaller of x's unit in the last place and the grid step,
// and the residual is below half a grid step, so it is a BF16 value.
typedef float rq_v2f __attribute__((ext_vector_type(2)));
template <class Fmt>
__device__ __forceinline__ uint4 residual8(uint4 q, uint2 c, uint32_t sb) {
  const float scale = e8m0_to_f32(sb);
  rq_v2f t[4];
  if constexpr (Fmt::kMantBits == 1) {
    t[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, scale, 0);
    t[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, scale, 1);
    t[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, scale, 2);
    t[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, scale, 3);
  } else {
    t[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, scale, false);
    t[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, scale, true);
    t[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, scale, false);
    t[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, scale, true);
  }
  const float d[8] = {t[0].x, t[0].y, t[1].x, t[1].y, t[2].x, t[2].y, t[3].x, t[3].y};
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xv = bf16_to_f32((e & 1) ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu);
    r[e] = __builtin_bit_cast(uint32_t, xv - d[e]) >> 16;
  }
  return pack8(r);
}

// Residual of one BF16 value (low half of v) against its own code under
// block scale byte sb, as a BF16 bit pattern: the element alone through the
// same scaled conversions as encode8 and residual8 (the conversion treats
// the two inputs of a pair independently, so the code is the one its block
// gave it), exact for the reason given at residual8.
template <class Fmt>
__device__ __forceinline__ uint32_t residual1(uint32_t v, uint32_t sb) {
  const float scale = e8m0_to_f32(sb);
  float d;
  if constexpr (Fmt::kMantBits == 1) {
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(rq_v2bf, v), scale, 0);
    const rq_v2f t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 0);
    d = t.x;
  } else {
    const rq_v2s c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((rq_v2s){0, 0}, __builtin_bit_cast(rq_v2bf, v), scale,
                                                               false);
    const rq_v2f t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(__builtin_bit_cast(uint32_t, c), scale, false);
    d = t.x;
  }
  return __builtin_bit_cast(uint32_t, bf16_to_f32(v) - d) >> 16;
}

// Encode 8 BF16 values with block scale byte sb and store them: FP4 -> one
// dword (element 2j in the low nibble of byte j), FP8 -> two dwords.
template <class Fmt>
__device__ __forceinline__ void encode_store8(uint4 q, uint32_t sb, uint8_t* dst) {
  store8<Fmt>(encode8<Fmt>(q, sb), dst);
}

}  // namespace rq
