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
// of dword i).
__device__ __forceinline__ uint32_t amax8(uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
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

// Encode 8 BF16 values with block scale byte sb and store them: FP4 -> one
// dword (element 2j in the low nibble of byte j), FP8 -> two dwords.
template <class Fmt>
__device__ __forceinline__ void encode_store8(uint4 q, uint32_t sb, uint8_t* dst) {
  store8<Fmt>(encode8<Fmt>(q, sb), dst);
}

}  // namespace rq
