// Row-wise kernels around the contractions:
//  * RMSNorm of the RAMP block input (RAMP page, section 4.2: the
//    surrounding operations stay BF16), optionally fused with the dynamic
//    block quantization of its output (Day-0 page, section V item 1:
//    quantize in the tail of the producing operator);
//  * the entropy / margin escalation gate over low-pass logits (escalation
//    article, setup paragraph);
//  * FP8 per-token-head-tile-128 KV quantize-on-write (Day-0 page, section
//    III.3.3 with the section V listing's amax/448 scale).
#include "rq_block.h"
#include "rq_internal.h"

namespace rq {

// One workgroup per row.  FMT 3: BF16 output; FMT 1/2: MX codes + scales
// (four consecutive threads own one 32-element block).
template <int FMT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ h, int64_t D, float eps,
                                                      uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const uint16_t* hr = h + row * D;
  const int chunks = (int)(D >> 3);
  float ss = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const uint4 q = *reinterpret_cast<const uint4*>(hr + c * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_to_f32(w[i] & 0xFFFFu), b = bf16_to_f32(w[i] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  const float total = block_sum(ss, sh);
  const float inv = 1.0f / sqrtf(total / (float)D + eps);
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const uint4 q = *reinterpret_cast<const uint4*>(hr + c * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t pw[4];  // the normalized pairs, BF16
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = pack_bf16(bf16_to_f32(w[i] & 0xFFFFu) * inv, bf16_to_f32(w[i] >> 16) * inv);
    const uint4 pk = make_uint4(pw[0], pw[1], pw[2], pw[3]);
    if constexpr (FMT == 3) {
      *reinterpret_cast<uint4*>(out + (row * D + c * 8) * 2) = pk;
    } else {
      using Fm = typename std::conditional<FMT == 1, FmtE2M1, FmtE4M3>::type;
      const uint32_t m = quad_max(amax8(pk));  // the quad is active together: chunks % 4 == 0
      const uint32_t sb = (uint32_t)(mx_block_exp<Fm>(m) + 127);
      if constexpr (FMT == 1)
        *reinterpret_cast<uint32_t*>(out + row * (D / 2) + c * 4) = cvt8_e2m1(pk, e8m0_to_f32(sb));
      else
        *reinterpret_cast<uint2*>(out + row * D + c * 8) = cvt8_e4m3(pk, e8m0_to_f32(sb));
      if ((c & 3) == 0) out_scales[row * (D / 32) + (c >> 2)] = (uint8_t)sb;
    }
  }
}

hipError_t launch_rmsnorm(int fmt, const uint16_t* h, int64_t rows, int64_t D, float eps, void* out,
                          uint8_t* out_scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint8_t* o = static_cast<uint8_t*>(out);
  if (fmt == 1)
    rmsnorm_kernel<1><<<(unsigned)rows, 256, 0, stream>>>(h, D, eps, o, out_scales);
  else if (fmt == 2)
    rmsnorm_kernel<2><<<(unsigned)rows, 256, 0, stream>>>(h, D, eps, o, out_scales);
  else
    rmsnorm_kernel<3><<<(unsigned)rows, 256, 0, stream>>>(h, D, eps, o, out_scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gate --
// One workgroup per token.  Pass 1: the two largest logits (m1 >= m2).
// Pass 2: Z = sum e^(z - m1) and W = sum (z - m1) e^(z - m1).  Then
// H = log Z - W / Z and p1 - p2 = (1 - e^(m2 - m1)) / Z.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  if (b1 > a1) {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  } else {
    a2 = fmaxf(a2, b1);
  }
}

__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ logits, int64_t V, float tau,
                                                   float delta, uint8_t* __restrict__ flags,
                                                   float* __restrict__ stats) {
  __shared__ float sh1[256], sh2[256];
  __shared__ float shs[4];
  const int64_t t = blockIdx.x;
  const uint16_t* z = logits + t * V;
  float m1 = -INFINITY, m2 = -INFINITY;
  for (int64_t i = threadIdx.x; i < V; i += 256) top2_merge(m1, m2, bf16_to_f32(z[i]), -INFINITY);
  sh1[threadIdx.x] = m1;
  sh2[threadIdx.x] = m2;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) {
      float a1 = sh1[threadIdx.x], a2 = sh2[threadIdx.x];
      top2_merge(a1, a2, sh1[threadIdx.x + s], sh2[threadIdx.x + s]);
      sh1[threadIdx.x] = a1;
      sh2[threadIdx.x] = a2;
    }
    __syncthreads();
  }
  const float M1 = sh1[0], M2 = sh2[0];
  float zs = 0.0f, ws = 0.0f;
  for (int64_t i = threadIdx.x; i < V; i += 256) {
    const float d = bf16_to_f32(z[i]) - M1;
    const float e = expf(d);
    zs += e;
    ws = fmaf(d, e, ws);
  }
  const float Z = block_sum(zs, shs);
  const float Wt = block_sum(ws, shs);
  if (threadIdx.x == 0) {
    const float H = logf(Z) - Wt / Z;
    const float gap = (1.0f - expf(M2 - M1)) / Z;
    flags[t] = (H > tau || gap < delta) ? 1 : 0;
    if (stats) {
      stats[2 * t] = H;
      stats[2 * t + 1] = gap;
    }
  }
}

hipError_t launch_gate(const uint16_t* logits, int64_t B, int64_t V, float tau, float delta, uint8_t* flags,
                       float* stats, hipStream_t stream) {
  gate_kernel<<<(unsigned)B, 256, 0, stream>>>(logits, V, tau, delta, flags, stats);
  return hipGetLastError();
}

// -------------------------------------------------------------- KV tiles --
// 16 threads per 128-element tile, 8 elements each; amax over the 16 lanes
// by xor-shuffles; float32 scale amax / 448 and float32 division.
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ x, int64_t tiles,
                                                       uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tile = gid >> 4;
  const int sub = (int)(gid & 15);
  const bool active = tile < tiles;
  uint4 q = make_uint4(0, 0, 0, 0);
  if (active) q = *reinterpret_cast<const uint4*>(x + tile * 128 + sub * 8);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 16));
  if (!active) return;
  const float amax = bf16_to_f32(m);
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  uint32_t c0 = 0, c1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = fminf(fmaxf(v[i] / scale, -448.0f), 448.0f);
    const float b = fminf(fmaxf(v[4 + i] / scale, -448.0f), 448.0f);
    c0 |= e4m3_encode_f32(a) << (8 * i);
    c1 |= e4m3_encode_f32(b) << (8 * i);
  }
  *reinterpret_cast<uint2*>(codes + tile * 128 + sub * 8) = make_uint2(c0, c1);
  if (sub == 0) scales[tile] = scale;
}

hipError_t launch_kv_quant(const uint16_t* x, int64_t T, int64_t H, int64_t D, uint8_t* codes, float* scales,
                           hipStream_t stream) {
  const int64_t tiles = T * H * (D / 128);
  if (tiles == 0) return hipSuccess;
  kv_quant_kernel<<<(unsigned)((tiles * 16 + 255) / 256), 256, 0, stream>>>(x, tiles, codes, scales);
  return hipGetLastError();
}

}  // namespace rq
