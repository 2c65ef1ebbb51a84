// Decode GEMV on 8-bit weights read through their top nibble, with 8-bit
// recompute of flagged tokens (Escalating Weight Precision Only When
// Decoding Becomes Uncertain, setup paragraph).  VALU only: no MFMA.
//
// Storage (made by pack_planes_kernel): two nibble planes, hi = w >> 4
// (two's complement) and lo = w & 15, tiled by 64 rows so that a wave's
// 64 lanes read 64 consecutive 16-byte chunks (one 32-element block of 64
// rows = 1 KiB, fully coalesced).  Inside a chunk, dword q holds the
// nibbles of k = 8q + 2j in bits 4j+3..4j and of k + 1 in bits 4j+19..4j+16,
// so one bit-field extract per element and one dword merge per pair give
// the BF16 pair (w_k, w_{k+1}) that v_dot2_f32_bf16 multiplies with the
// token pair (x_k, x_{k+1}) -- a plain aligned dword of the BF16 row.
//
// Work split: a workgroup owns 64 rows; its four waves take interleaved
// 32-blocks of K; per block each lane turns its 16 bytes into 16 exact BF16
// pairs once and reuses them for every token (x comes through the scalar
// cache: the address is wave-uniform).  FP32 block partials are scaled by
// the block's FP16 scale (x16 for the top nibble, exact) and accumulated;
// the four waves' sums are added in a fixed order through LDS.
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int sbfe(uint32_t v, int off, int w) {
  return __builtin_amdgcn_sbfe((int)v, off, w);
}
// Two small exact integers -> packed BF16 pair (truncation is exact).
__device__ __forceinline__ bf16x2 pack_ints(int a, int b) {
  const uint32_t fa = __builtin_bit_cast(uint32_t, (float)a);
  const uint32_t fb = __builtin_bit_cast(uint32_t, (float)b);
  return __builtin_bit_cast(bf16x2, (fa >> 16) | (fb & 0xFFFF0000u));
}
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }
__device__ __forceinline__ float f16_to_f32(uint16_t s) { return (float)__builtin_bit_cast(_Float16, s); }

// The 16 pairs of a hi-plane chunk: pair p = 4q + j covers k = 8q+2j, +1.
__device__ __forceinline__ void unpack_hi(const uint4 d, bf16x2 wp[16]) {
  const uint32_t dq[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) wp[4 * q + j] = pack_ints(sbfe(dq[q], 4 * j, 4), sbfe(dq[q], 16 + 4 * j, 4));
}

// Full 8-bit weights from the hi and lo chunks: byte (hi << 4 | lo) is the
// int8 weight.  E0 bytes hold nibble positions 0,2,4,6 and E1 positions
// 1,3,5,7; pair j combines positions j and j + 4.
__device__ __forceinline__ void unpack_full(const uint4 dh, const uint4 dl, bf16x2 wp[16]) {
  const uint32_t h[4] = {dh.x, dh.y, dh.z, dh.w};
  const uint32_t l[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t e0 = ((h[q] << 4) & 0xF0F0F0F0u) | (l[q] & 0x0F0F0F0Fu);
    const uint32_t e1 = (h[q] & 0xF0F0F0F0u) | ((l[q] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = (j & 1) ? e1 : e0;
      wp[4 * q + j] = pack_ints(sbfe(e, 8 * (j >> 1), 8), sbfe(e, 8 * (2 + (j >> 1)), 8));
    }
  }
}

template <int TB>
__global__ __launch_bounds__(256) void gemv_low_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                       const uint8_t* __restrict__ hi,
                                                       const uint16_t* __restrict__ sc, uint16_t* __restrict__ y) {
  __shared__ float red[4][TB][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int nb = K >> 5;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + (size_t)tile * nb * 64 + lane;
  const uint16_t* sp = sc + (size_t)tile * nb * 64 + lane;
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;

  for (int b = wave; b < nb; b += 4) {
    const uint4 d = hp[(size_t)b * 64];
    const float s = f16_to_f32(sp[(size_t)b * 64]) * 16.0f;
    bf16x2 wp[16];
    unpack_hi(d, wp);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int tt = t < B ? t : B - 1;
      const uint32_t* xt = x32 + ((size_t)tt * K + 32 * (size_t)b) / 2;
      float blk = 0.0f;
#pragma unroll
      for (int p = 0; p < 16; ++p) blk = __builtin_amdgcn_fdot2_f32_bf16(wp[p], as_bf16x2(xt[p]), blk, false);
      acc[t] = fmaf(blk, s, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int o = threadIdx.x; o < TB * 64; o += 256) {
    const int t = o >> 6, l = o & 63;
    const int n = tile * 64 + l;
    if (t < B && n < N) {
      const float v = ((red[0][t][l] + red[1][t][l]) + red[2][t][l]) + red[3][t][l];
      y[(size_t)t * N + n] = (uint16_t)f32_to_bf16(v);
    }
  }
}

template <int TB>
__global__ __launch_bounds__(256) void gemv_escalate_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                            const uint8_t* __restrict__ hi,
                                                            const uint8_t* __restrict__ lo,
                                                            const uint16_t* __restrict__ sc,
                                                            const uint8_t* __restrict__ flags,
                                                            uint16_t* __restrict__ y) {
  __shared__ float red[4][TB][64];
  uint32_t fmask = 0;
  for (int t = 0; t < B; ++t) fmask |= (flags[t] != 0 ? 1u : 0u) << t;
  fmask = __builtin_amdgcn_readfirstlane(fmask);
  if (fmask == 0) return;  // nothing flagged: no weight traffic
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int nb = K >> 5;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + (size_t)tile * nb * 64 + lane;
  const uint4* lp = reinterpret_cast<const uint4*>(lo) + (size_t)tile * nb * 64 + lane;
  const uint16_t* sp = sc + (size_t)tile * nb * 64 + lane;
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;

  for (int b = wave; b < nb; b += 4) {
    const uint4 dh = hp[(size_t)b * 64];
    const uint4 dl = lp[(size_t)b * 64];
    const float s = f16_to_f32(sp[(size_t)b * 64]);
    bf16x2 wp[16];
    unpack_full(dh, dl, wp);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (!((fmask >> t) & 1u)) continue;  // wave-uniform branch
      const uint32_t* xt = x32 + ((size_t)t * K + 32 * (size_t)b) / 2;
      float blk = 0.0f;
#pragma unroll
      for (int p = 0; p < 16; ++p) blk = __builtin_amdgcn_fdot2_f32_bf16(wp[p], as_bf16x2(xt[p]), blk, false);
      acc[t] = fmaf(blk, s, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int o = threadIdx.x; o < TB * 64; o += 256) {
    const int t = o >> 6, l = o & 63;
    const int n = tile * 64 + l;
    if (t < B && ((fmask >> t) & 1u) && n < N) {
      const float v = ((red[0][t][l] + red[1][t][l]) + red[2][t][l]) + red[3][t][l];
      y[(size_t)t * N + n] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// One thread per (padded row, 32-block): 32 int8 weights -> one 16-byte
// chunk of each plane in the tiled layout, plus the tiled scale.
__global__ __launch_bounds__(256) void pack_planes_kernel(const int8_t* __restrict__ w,
                                                          const uint16_t* __restrict__ sc, int64_t N, int64_t K,
                                                          int64_t Np, uint8_t* __restrict__ hi,
                                                          uint8_t* __restrict__ lo, uint16_t* __restrict__ sct) {
  const int64_t nb = K >> 5;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= Np * nb) return;
  const int64_t n = gid / nb, b = gid - n * nb;
  uint32_t hq[4] = {0, 0, 0, 0}, lq[4] = {0, 0, 0, 0};
  uint16_t s = 0;
  if (n < N) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(w) + n * K + b * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wa = src[8 * q + 2 * j], wb = src[8 * q + 2 * j + 1];
        hq[q] |= ((wa >> 4) & 0xFu) << (4 * j) | ((wb >> 4) & 0xFu) << (16 + 4 * j);
        lq[q] |= (wa & 0xFu) << (4 * j) | (wb & 0xFu) << (16 + 4 * j);
      }
    s = sc[n * nb + b];
  }
  const int64_t chunk = ((n >> 6) * nb + b) * 64 + (n & 63);
  reinterpret_cast<uint4*>(hi)[chunk] = make_uint4(hq[0], hq[1], hq[2], hq[3]);
  reinterpret_cast<uint4*>(lo)[chunk] = make_uint4(lq[0], lq[1], lq[2], lq[3]);
  sct[chunk] = s;
}

hipError_t launch_pack_nibble_planes(const int8_t* w, const uint16_t* scales, int64_t N, int64_t K,
                                     uint8_t* hi, uint8_t* lo, uint16_t* scales_tiled, hipStream_t stream) {
  const int64_t Np = (N + 63) / 64 * 64;
  const int64_t threads = Np * (K / 32);
  if (threads == 0) return hipSuccess;
  pack_planes_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(w, scales, N, K, Np, hi, lo,
                                                                            scales_tiled);
  return hipGetLastError();
}

hipError_t launch_gemv_low(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                           const uint16_t* scales, uint16_t* y, hipStream_t stream) {
  const unsigned g = (unsigned)((N + 63) / 64);
  if (g == 0) return hipSuccess;
  const int b = (int)B, k = (int)K, n = (int)N;
  if (B <= 1)
    gemv_low_kernel<1><<<g, 256, 0, stream>>>(x, b, k, n, hi, scales, y);
  else if (B <= 2)
    gemv_low_kernel<2><<<g, 256, 0, stream>>>(x, b, k, n, hi, scales, y);
  else if (B <= 4)
    gemv_low_kernel<4><<<g, 256, 0, stream>>>(x, b, k, n, hi, scales, y);
  else if (B <= 8)
    gemv_low_kernel<8><<<g, 256, 0, stream>>>(x, b, k, n, hi, scales, y);
  else
    gemv_low_kernel<16><<<g, 256, 0, stream>>>(x, b, k, n, hi, scales, y);
  return hipGetLastError();
}

hipError_t launch_gemv_escalate(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                                const uint8_t* lo, const uint16_t* scales, const uint8_t* flags, uint16_t* y,
                                hipStream_t stream) {
  const unsigned g = (unsigned)((N + 63) / 64);
  if (g == 0) return hipSuccess;
  const int b = (int)B, k = (int)K, n = (int)N;
  if (B <= 2)
    gemv_escalate_kernel<2><<<g, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y);
  else if (B <= 4)
    gemv_escalate_kernel<4><<<g, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y);
  else if (B <= 8)
    gemv_escalate_kernel<8><<<g, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y);
  else
    gemv_escalate_kernel<16><<<g, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y);
  return hipGetLastError();
}

}  // namespace rq
