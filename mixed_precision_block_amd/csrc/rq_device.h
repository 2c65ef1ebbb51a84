// Device-side number-format helpers for the gfx950 kernels.
//
// Block scale (Day 0 LLM Inference Support, section V per-group listing and
// section III.3.2 power-of-two scales): the block exponent is the smallest
// e with amax <= Qmax * 2^e.  On BF16 bits amax = (1 + f/128) * 2^(E-127);
// Qmax = 1.5 * 2^2 (E2M1) or 1.75 * 2^8 (E4M3), so
//   e = (E - 127) - emax + (f > fq),  (emax, fq) = (2, 64) or (8, 96),
// clamped below at -127 (a subnormal amax always clamps).
//
// Element encode: round-to-nearest-even of x * 2^-e onto the E2M1 / E4M3FN
// grid, done on integers from the BF16 bits so it is exact for every input
// (no float multiply, no denormal flushing).  The value is M * 2^s with an
// integer significand M <= 255; in the binade of k = floor(log2 v)
// (clamped to the format's smallest normal exponent) the grid step is
// 2^(k - mbits), so the code is ((k - emin) << mbits) + RNE(v / step).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define RQ_HD __host__ __device__ __forceinline__

namespace rq {

struct FmtE2M1 {
  static constexpr int kMantBits = 1;
  static constexpr int kEmin = 0;       // smallest normal: 2^0
  static constexpr uint32_t kMaxCode = 7;
  static constexpr int kSignShift = 3;
  static constexpr int kEmax = 2;       // Qmax = 1.5 * 2^2
  static constexpr int kFq = 64;
};
struct FmtE4M3 {
  static constexpr int kMantBits = 3;
  static constexpr int kEmin = -6;      // smallest normal: 2^-6
  static constexpr uint32_t kMaxCode = 0x7E;
  static constexpr int kSignShift = 7;
  static constexpr int kEmax = 8;       // Qmax = 1.75 * 2^8
  static constexpr int kFq = 96;
};

RQ_HD float bf16_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// Round a finite float to BF16, nearest-even.
RQ_HD uint32_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// SiLU(z) = z / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal (each within about an ulp of fp32; the GEMM epilogues round
// the result to BF16).  Very negative z gives e^-z = inf and a zero
// reciprocal: SiLU tends to -0, as it should.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// Two floats to packed BF16 (lo in bits 15:0) by the hardware conversion
// (v_cvt_pk_bf16_f32): round to nearest even, the same bits as f32_to_bf16
// for finite values.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, (bf16x2_t){(__bf16)lo, (__bf16)hi});
}

// Block exponent from the 15-bit magnitude bits of the block amax.
template <class Fmt>
RQ_HD int mx_block_exp(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  int E = (int)(amax_bits >> 7);
  if (E == 0) return -127;
  int f = (int)(amax_bits & 0x7F);
  int e = (E - 127) - Fmt::kEmax + (f > Fmt::kFq ? 1 : 0);
  return e < -127 ? -127 : e;
}

// Magnitude code of |x| * 2^-e for BF16 magnitude bits xb.
template <class Fmt>
RQ_HD uint32_t mx_encode_mag(uint32_t xb, int e) {
  if (xb == 0) return 0;
  uint32_t Ex = xb >> 7;
  uint32_t M = Ex ? (0x80u | (xb & 0x7Fu)) : (xb & 0x7Fu);
  int s = (Ex ? (int)Ex - 134 : -133) - e;  // value = M * 2^s
  int L = 32 - __builtin_clz(M);                     // bit length of M
  int k = L - 1 + s;                          // floor(log2 value)
  if (k < Fmt::kEmin) k = Fmt::kEmin;
  int r = (k - Fmt::kMantBits) - s;           // right shift to the grid step
  uint32_t n;
  if (r <= 0) {
    n = M << (-r);
  } else if (r >= 9) {
    n = 0;  // M < 2^8: below half a step
  } else {
    n = M >> r;
    uint32_t rem = M & ((1u << r) - 1u);
    uint32_t half = 1u << (r - 1);
    n += (rem > half || (rem == half && (n & 1u))) ? 1u : 0u;
  }
  uint32_t code = ((uint32_t)(k - Fmt::kEmin) << Fmt::kMantBits) + n;
  return code > Fmt::kMaxCode ? Fmt::kMaxCode : code;
}

template <class Fmt>
RQ_HD uint32_t mx_encode(uint32_t xbits, int e) {
  return mx_encode_mag<Fmt>(xbits & 0x7FFFu, e) | (((xbits >> 15) & 1u) << Fmt::kSignShift);
}

// Exact value of a magnitude code (without scale), as float.
RQ_HD float e2m1_mag_value(uint32_t c) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  uint32_t ex = c >> 1, m = c & 1u;
  return ex == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)ex - 1);
}
RQ_HD float e4m3_mag_value(uint32_t c) {
  uint32_t ex = c >> 3, m = c & 7u;
  return ex == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf(1.0f + 0.125f * (float)m, (int)ex - 7);
}

template <class Fmt>
RQ_HD float mx_mag_value(uint32_t c);
template <>
RQ_HD float mx_mag_value<FmtE2M1>(uint32_t c) { return e2m1_mag_value(c); }
template <>
RQ_HD float mx_mag_value<FmtE4M3>(uint32_t c) { return e4m3_mag_value(c); }

}  // namespace rq
