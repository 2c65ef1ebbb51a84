// gfx950 scaled conversions from BF16 to the MX element formats (device
// only).  v_cvt_scalef32_pk_{fp4,fp8}_bf16 divides each of two BF16 inputs
// by a float scale and rounds to nearest-even onto the E2M1 / E4M3FN grid,
// keeping the sign of values that round to zero.  For every input the block
// scale covers (|x| <= Qmax 2^e, the only inputs the block quantizer
// presents) this is the element encode of the Day 0 page's per-group
// listing (section V) with the power-of-two scale of section III.3.2, the
// same codes as the integer encoder mx_encode in rq_device.h.  The scale
// is the block's E8M0 value as a float: 2^(b - 127), which for b = 0 is the
// float subnormal 2^-127.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

typedef short rq_v2s __attribute__((ext_vector_type(2)));
typedef __bf16 rq_v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 rq_v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b ? b << 23 : 0x00400000u);
}

// Eight BF16 values (element 2i in the low half of dword i) to E2M1 codes:
// element k in nibble k of the result.
__device__ __forceinline__ uint32_t cvt8_e2m1(uint4 q, float scale) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(rq_v2bf, q.x), scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(rq_v2bf, q.y), scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(rq_v2bf, q.z), scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(rq_v2bf, q.w), scale, 3);
  return w;
}

// Eight BF16 values to E4M3FN codes: element k in byte k of the pair.
__device__ __forceinline__ uint2 cvt8_e4m3(uint4 q, float scale) {
  rq_v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((rq_v2s){0, 0}, __builtin_bit_cast(rq_v2bf, q.x), scale, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(rq_v2bf, q.y), scale, true);
  rq_v2s hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((rq_v2s){0, 0}, __builtin_bit_cast(rq_v2bf, q.z), scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(rq_v2bf, q.w), scale, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Eight E4M3FN codes (byte k of the pair = element k) times a float scale
// to BF16, by v_cvt_scalef32_pk_bf16_fp8.  Every E4M3 value has four
// significant bits, so the result is the exact product whenever it lies in
// BF16's normal range (block exponents from -117 up; the quantizer's
// exponents for BF16 inputs never reach the top of the range).
__device__ __forceinline__ rq_v8bf deq8_e4m3(uint32_t lo, uint32_t hi, float scale) {
  const rq_v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  const rq_v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  const rq_v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  const rq_v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  return rq_v8bf{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

}  // namespace rq
