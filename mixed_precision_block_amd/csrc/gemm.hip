// Block-scaled GEMM on gfx950 matrix cores: Y[M x N] = A . W^T, K-major
// operands, FP32 accumulation.
//
// MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 consumes 32 K-elements per lane
// together with that lane's E8M0 block scale, so the block scales of the
// ARCQuant unified GEMM and of the Day-0 page (section V item 3: scales
// applied inside the multiply-accumulate) never produce a dequantized
// intermediate in memory; E2M1 products are exact.  MXFP8: the same
// instruction on FP8 truncates products inside runs of 8 K terms (about
// 4e-5 relative on normal data), so each lane dequantizes its E4M3 codes
// with their block scale to BF16 in registers (exact) and the BF16
// instruction accumulates in FP32; the FP8 instruction itself is FMT 4.
// BF16: v_mfma_f32_32x32x16_bf16 on the same tiling (the reference-precision
// steps of RAMP, section 4.2).
//
// Operand layout per MFMA (pinned by the single-tile GPU parity test):
//   lane l supplies row (l % 32) of a 64-deep MX slice plus the E8M0 byte
//   of (row, block l / 32).  FP4: the lane's 16 bytes are K [32h, 32h+32)
//   with h = l / 32.  FP8: the matrix core takes the first 16 bytes of both
//   lane halves as block 0 and the last 16 bytes as block 1, so lane half h
//   carries K [16h, 16h+16) then K [32+16h, 32+16h+16).  BF16: lane l
//   supplies 8 elements at K offset 8 h of a 16-deep slice.  Accumulator
//   element r of lane l is D[8 (r / 4) + 4 h + r % 4][l % 32].
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile; its four waves
// each own a 64 x 64 quadrant (2 x 2 MFMA tiles).  Each K step stages a
// 128-row slice of A and of W in LDS (rows padded by 16 bytes so the
// 16-byte reads of 8 consecutive lanes hit distinct banks), double
// buffered through registers: the next slice's global loads are in flight
// while the current one feeds the MFMAs.  Tails in M, N and K are
// zero-filled (zero codes with scale byte 127 contribute nothing).
#include "rq_cvt.h"
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int FMT>
struct GemmTraits;
template <>
struct GemmTraits<1> {  // MXFP4
  static constexpr int kStepElems = 128, kRowBytes = 64, kKK = 2, kOpBytes = 16, kKKBytes = 32;
  static constexpr int kCbsz = 4;
  static constexpr bool kScaled = true;
};
template <>
struct GemmTraits<2> {  // MXFP8 (E4M3)
  static constexpr int kStepElems = 128, kRowBytes = 128, kKK = 2, kOpBytes = 32, kKKBytes = 64;
  static constexpr int kCbsz = 0;
  static constexpr bool kScaled = true;
};
template <>
struct GemmTraits<4> : GemmTraits<2> {};  // MXFP8 on the FP8 scaled MFMA
template <>
struct GemmTraits<3> {  // BF16
  static constexpr int kStepElems = 64, kRowBytes = 128, kKK = 4, kOpBytes = 16, kKKBytes = 32;
  static constexpr int kCbsz = 0;
  static constexpr bool kScaled = false;
};

constexpr int kTile = 128;

template <int FMT, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                                                   const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws,
                                                   int M, int N, int K, void* __restrict__ Y) {
  using T = GemmTraits<FMT>;
  constexpr int RB = T::kRowBytes;
  constexpr int LDSR = RB + 16;
  constexpr int CH = RB / 16;                 // 16-byte chunks per row per step
  constexpr int LOADS = kTile * CH / 256;     // chunks per thread per operand
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kTile * LDSR];
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][kTile * LDSR];
  __shared__ __attribute__((aligned(16))) uint8_t sS[2][2 * kTile * 4];  // A then W scale bytes

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTile, n0 = blockIdx.x * kTile;
  constexpr bool kF8 = FMT == 2 || FMT == 4;
  const int64_t ld = FMT == 1 ? K / 2 : (kF8 ? K : 2 * (int64_t)K);  // row bytes
  const int ksb = K / 32;
  const int nk = (K + T::kStepElems - 1) / T::kStepElems;

  uint4 ra[LOADS], rw[LOADS];
  uint32_t rs = 0x7F7F7F7Fu;

  auto gload = [&](int kt) {
    const int64_t kb0 = (int64_t)kt * RB;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + i * 256, r = c / CH, cc = c % CH;
      const int64_t kb = kb0 + cc * 16;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M && kb < ld) ? *reinterpret_cast<const uint4*>(A + gm * ld + kb) : make_uint4(0, 0, 0, 0);
      rw[i] = (gn < N && kb < ld) ? *reinterpret_cast<const uint4*>(W + gn * ld + kb) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (T::kScaled) {
      const int r = tid & 127;
      const bool isw = tid >= 128;
      const int g = (isw ? n0 : m0) + r;
      const uint8_t* sp = (isw ? Ws : As) + (int64_t)g * ksb;
      uint32_t s = 0x7F7F7F7Fu;
      if (g < (isw ? N : M)) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int kb = kt * 4 + b;
          const uint32_t byte = kb < ksb ? sp[kb] : 127u;
          s = (s & ~(0xFFu << (8 * b))) | (byte << (8 * b));
        }
      }
      rs = s;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + i * 256, r = c / CH, cc = c % CH;
      *reinterpret_cast<uint4*>(&sA[buf][r * LDSR + cc * 16]) = ra[i];
      *reinterpret_cast<uint4*>(&sW[buf][r * LDSR + cc * 16]) = rw[i];
    }
    if constexpr (T::kScaled) *reinterpret_cast<uint32_t*>(&sS[buf][tid * 4]) = rs;
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  gload(0);
  sstore(0);
  __syncthreads();

  const int half = lane >> 5, lrow = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < T::kKK; ++kk) {
      v8i a_op[2], b_op[2];
      v8bf a_bf[2], b_bf[2];
      int sa[2], sb[2];
      float fa[2][2], fb[2][2];  // exact MXFP8: both block scales of the slice
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ar = wm * 64 + i * 32 + lrow;
        const int br = wn * 64 + i * 32 + lrow;
        // FP8 lane halves interleave at 16 bytes (see the layout note above)
        constexpr int kHalfStride = kF8 ? 16 : T::kOpBytes;
        constexpr int kSecond = kF8 ? 32 : 16;
        const uint8_t* pa = &sA[buf][ar * LDSR + kk * T::kKKBytes + half * kHalfStride];
        const uint8_t* pb = &sW[buf][br * LDSR + kk * T::kKKBytes + half * kHalfStride];
        if constexpr (FMT == 3) {
          a_bf[i] = *reinterpret_cast<const v8bf*>(pa);
          b_bf[i] = *reinterpret_cast<const v8bf*>(pb);
        } else {
          const uint4 a0 = *reinterpret_cast<const uint4*>(pa);
          const uint4 b0 = *reinterpret_cast<const uint4*>(pb);
          uint4 a1 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);
          if constexpr (T::kOpBytes == 32) {
            a1 = *reinterpret_cast<const uint4*>(pa + kSecond);
            b1 = *reinterpret_cast<const uint4*>(pb + kSecond);
          }
          a_op[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          b_op[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          sa[i] = sS[buf][ar * 4 + kk * 2 + half];
          sb[i] = sS[buf][kTile * 4 + br * 4 + kk * 2 + half];
          if constexpr (FMT == 2) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              fa[i][b] = e8m0_to_f32(sS[buf][ar * 4 + kk * 2 + b]);
              fb[i][b] = e8m0_to_f32(sS[buf][kTile * 4 + br * 4 + kk * 2 + b]);
            }
          }
        }
      }
      if constexpr (FMT == 2) {
        // exact MXFP8: BF16 MFMA q takes 8 codes per lane (dwords 2 (q % 2),
        // +1 of 16-byte chunk q / 2, scaled by block q / 2), dequantized to
        // BF16; the same K for both operands, so the four cover the slice
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rq_v8bf da[2], dw[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int lo = q / 2 ? 4 : 0;
            const int d0 = lo + 2 * (q % 2);
            da[i] = deq8_e4m3((uint32_t)a_op[i][d0], (uint32_t)a_op[i][d0 + 1], fa[i][q / 2]);
            dw[i] = deq8_e4m3((uint32_t)b_op[i][d0], (uint32_t)b_op[i][d0 + 1], fb[i][q / 2]);
          }
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[i], dw[j], acc[i][j], 0, 0, 0);
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (FMT == 3)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_bf[i], b_bf[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a_op[i], b_op[j], acc[i][j], T::kCbsz,
                                                                         T::kCbsz, 0, sa[i], 0, sb[j]);
        }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column n, rows 8 (r/4) + 4 half + r%4 of each tile.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + lrow;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m >= M) continue;
        const float v = acc[i][j][r];
        const int64_t o = (int64_t)m * N + n;
        if constexpr (EPI == kEpiStoreF32) {
          reinterpret_cast<float*>(Y)[o] = v;
        } else if constexpr (EPI == kEpiStoreBf16) {
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(v);
        } else if constexpr (EPI == kEpiSiluBf16) {
          const float z = bf16_to_f32(f32_to_bf16(v));
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(silu_f32(z));
        } else {
          uint16_t* h = reinterpret_cast<uint16_t*>(Y);
          const float sum = bf16_to_f32(h[o]) + bf16_to_f32(f32_to_bf16(v));
          h[o] = (uint16_t)f32_to_bf16(sum);
        }
      }
    }
}

template <int FMT>
static hipError_t launch_fmt(int epi, const void* a, const uint8_t* as, const void* w, const uint8_t* ws,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((M + kTile - 1) / kTile));
  const uint8_t* A = static_cast<const uint8_t*>(a);
  const uint8_t* W = static_cast<const uint8_t*>(w);
  switch (epi) {
    case kEpiStoreBf16:
      gemm_kernel<FMT, kEpiStoreBf16><<<grid, 256, 0, stream>>>(A, as, W, ws, (int)M, (int)N, (int)K, y);
      break;
    case kEpiStoreF32:
      gemm_kernel<FMT, kEpiStoreF32><<<grid, 256, 0, stream>>>(A, as, W, ws, (int)M, (int)N, (int)K, y);
      break;
    case kEpiSiluBf16:
      gemm_kernel<FMT, kEpiSiluBf16><<<grid, 256, 0, stream>>>(A, as, W, ws, (int)M, (int)N, (int)K, y);
      break;
    default:
      gemm_kernel<FMT, kEpiResAddBf16><<<grid, 256, 0, stream>>>(A, as, W, ws, (int)M, (int)N, (int)K, y);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                       const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                       hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (gemm_pipe_supported(fmt, M, N, K))
    return launch_gemm_pipe(fmt, epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  return launch_gemm_basic(fmt, epi, a, a_scales, w, w_scales, M, N, K, y, stream);
}

hipError_t launch_gemm_basic(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                             const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                             hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fmt == 1) return launch_fmt<1>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  if (fmt == 2) return launch_fmt<2>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  if (fmt == 4) return launch_fmt<4>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  return launch_fmt<3>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
}

}  // namespace rq
