// Row-wise kernels around the contractions:
//  * RMSNorm of the RAMP block input (RAMP page, section 4.2: the
//    surrounding operations stay BF16), optionally fused with the dynamic
//    block quantization of its output (Day-0 page, section V item 1:
//    quantize in the tail of the producing operator);
//  * the entropy / margin escalation gate over low-pass logits (escalation
//    article, setup paragraph);
//  * FP8 per-token-head-tile-128 KV quantize-on-write (Day-0 page, section
//    III.3.3 with the section V listing's amax/448 scale).
#include <algorithm>
#include <mutex>

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

// Rows of up to 4096 elements: one wave per row, four rows per workgroup,
// the row held in registers between the two passes and no workgroup
// barrier.  Lane l plays threads l, l + 64, l + 128 and l + 192 of
// rmsnorm_kernel: it keeps their partial sums of squares apart, each over
// the same chunks in the same order, and adds the four wave sums in that
// kernel's order, so the two give the same bits.
template <int FMT, int MC>
__global__ __launch_bounds__(256) void rmsnorm_wave_kernel(const uint16_t* __restrict__ h, int64_t rows, int64_t D,
                                                           float eps, uint8_t* __restrict__ out,
                                                           uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t* hr = h + row * D;
  const int chunks = (int)(D >> 3);
  uint4 q[4][MC];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int c = 256 * m + 64 * k + lane;
      q[k][m] = c < chunks ? *reinterpret_cast<const uint4*>(hr + c * 8) : make_uint4(0, 0, 0, 0);
    }
  float part[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float ss = 0.0f;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      if (256 * m + 64 * k + lane >= chunks) continue;
      const uint32_t w[4] = {q[k][m].x, q[k][m].y, q[k][m].z, q[k][m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_to_f32(w[i] & 0xFFFFu), b = bf16_to_f32(w[i] >> 16);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
    part[k] = wave_sum(ss);
  }
  const float total = ((part[0] + part[1]) + part[2]) + part[3];
  const float inv = 1.0f / sqrtf(total / (float)D + eps);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int c = 256 * m + 64 * k + lane;
      if (256 * m + 64 * k >= chunks) continue;  // wave-uniform: no chunk of this round is in the row
      const uint32_t w[4] = {q[k][m].x, q[k][m].y, q[k][m].z, q[k][m].w};
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[i] = pack_bf16(bf16_to_f32(w[i] & 0xFFFFu) * inv, bf16_to_f32(w[i] >> 16) * inv);
      const uint4 pk = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      if constexpr (FMT == 3) {
        if (c < chunks) *reinterpret_cast<uint4*>(out + (row * D + c * 8) * 2) = pk;
      } else {
        // a quad of lanes owns one 32-block; with chunks % 4 == 0 the quad is in or out together
        using Fm = typename std::conditional<FMT == 1, FmtE2M1, FmtE4M3>::type;
        const uint32_t mx = quad_max(amax8(pk));
        const uint32_t sb = (uint32_t)(mx_block_exp<Fm>(mx) + 127);
        if (c < chunks) {
          if constexpr (FMT == 1)
            *reinterpret_cast<uint32_t*>(out + row * (D / 2) + c * 4) = cvt8_e2m1(pk, e8m0_to_f32(sb));
          else
            *reinterpret_cast<uint2*>(out + row * D + c * 8) = cvt8_e4m3(pk, e8m0_to_f32(sb));
          if ((c & 3) == 0) out_scales[row * (D / 32) + (c >> 2)] = (uint8_t)sb;
        }
      }
    }
}

template <int FMT>
static hipError_t launch_rmsnorm_f(const uint16_t* h, int64_t rows, int64_t D, float eps, uint8_t* o,
                                   uint8_t* out_scales, hipStream_t stream) {
  const unsigned g4 = (unsigned)((rows + 3) / 4);
  if (D <= 2048)
    rmsnorm_wave_kernel<FMT, 1><<<g4, 256, 0, stream>>>(h, rows, D, eps, o, out_scales);
  else if (D <= 4096)
    rmsnorm_wave_kernel<FMT, 2><<<g4, 256, 0, stream>>>(h, rows, D, eps, o, out_scales);
  else
    rmsnorm_kernel<FMT><<<(unsigned)rows, 256, 0, stream>>>(h, D, eps, o, out_scales);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int fmt, const uint16_t* h, int64_t rows, int64_t D, float eps, void* out,
                          uint8_t* out_scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint8_t* o = static_cast<uint8_t*>(out);
  if (fmt == 1) return launch_rmsnorm_f<1>(h, rows, D, eps, o, out_scales, stream);
  if (fmt == 2) return launch_rmsnorm_f<2>(h, rows, D, eps, o, out_scales, stream);
  return launch_rmsnorm_f<3>(h, rows, D, eps, o, out_scales, stream);
}

// ------------------------------------------------------------------ gate --
// Softmax entropy and top-1 / top-2 margin from a row's two largest logits
// m1 >= m2, Z = sum e^(z - m1) and W = sum (z - m1) e^(z - m1):
// H = log Z - W / Z and p1 - p2 = (1 - e^(m2 - m1)) / Z.  A row splits into
// ranges whose statistics (each relative to its own m1) merge exactly:
// with M the larger maximum, Z = sum_g Z_g e^(m1_g - M) and
// W = sum_g e^(m1_g - M) (W_g + (m1_g - M) Z_g).
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  if (b1 > a1) {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  } else {
    a2 = fmaxf(a2, b1);
  }
}

// Visits elements [lo, hi) of a BF16 row with the 256 threads of a
// workgroup: the part from the first 16-byte boundary on in 8-element
// vector loads, the few elements before it and after the last full vector
// one per thread.
template <typename F>
__device__ __forceinline__ void gate_visit(const uint16_t* __restrict__ z, int64_t lo, int64_t hi, F&& fn) {
  const int64_t head = ((16 - (reinterpret_cast<uintptr_t>(z + lo) & 15)) & 15) / 2;
  const int64_t v0 = min(hi, lo + head);
  const int64_t nv = (hi - v0) / 8, v1 = v0 + nv * 8;
  const int tid = (int)threadIdx.x;
  if (lo + tid < v0) fn(bf16_to_f32(z[lo + tid]));
  if (v1 + tid < hi) fn(bf16_to_f32(z[v1 + tid]));
  const uint4* zv = reinterpret_cast<const uint4*>(z + v0);
  for (int64_t c = tid; c < nv; c += 256) {
    const uint4 q = zv[c];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fn(bf16_to_f32(w[i] & 0xFFFFu));
      fn(bf16_to_f32(w[i] >> 16));
    }
  }
}

// The statistics of z[lo, hi) (non-empty), computed by a 256-thread
// workgroup and returned to every thread; two passes, the second reading
// the range again (from cache).
__device__ __forceinline__ float4 gate_range(const uint16_t* __restrict__ z, int64_t lo, int64_t hi) {
  __shared__ float s1[4], s2[4], ss[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m1 = -INFINITY, m2 = -INFINITY;
  gate_visit(z, lo, hi, [&](float v) {
    m2 = fmaxf(m2, fminf(m1, v));
    m1 = fmaxf(m1, v);
  });
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) top2_merge(m1, m2, __shfl_xor(m1, o, 64), __shfl_xor(m2, o, 64));
  if (lane == 0) s1[wave] = m1, s2[wave] = m2;
  __syncthreads();
  float M1 = s1[0], M2 = s2[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) top2_merge(M1, M2, s1[w], s2[w]);
  float zs = 0.0f, ws = 0.0f;
  gate_visit(z, lo, hi, [&](float v) {
    const float d = v - M1;
    const float e = expf(d);
    zs += e;
    ws = fmaf(d, e, ws);
  });
  const float Z = block_sum(zs, ss);
  const float W = block_sum(ws, ss);
  return make_float4(M1, M2, Z, W);
}

__device__ __forceinline__ void gate_finish(float M1, float M2, float Z, float W, float tau, float delta,
                                            uint8_t* __restrict__ flags, float* __restrict__ stats, int64_t t) {
  const float H = logf(Z) - W / Z;
  const float gap = (1.0f - expf(M2 - M1)) / Z;
  flags[t] = (H > tau || gap < delta) ? 1 : 0;
  if (stats) {
    stats[2 * t] = H;
    stats[2 * t + 1] = gap;
  }
}

// Without a workspace: one workgroup per token over its whole row.
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ logits, int64_t V, float tau,
                                                   float delta, uint8_t* __restrict__ flags,
                                                   float* __restrict__ stats) {
  const int64_t t = blockIdx.x;
  const float4 r = gate_range(logits + t * V, 0, V);
  if (threadIdx.x == 0) gate_finish(r.x, r.y, r.z, r.w, tau, delta, flags, stats, t);
}

// With a workspace: workgroup (g, t) takes range g of token t's row and
// stores its statistics; gate_merge_kernel (one wave per token) combines
// the token's ranges in a fixed order.
__global__ __launch_bounds__(256) void gate_part_kernel(const uint16_t* __restrict__ logits, int64_t V,
                                                        int64_t chunk, float4* __restrict__ parts) {
  const int64_t g = blockIdx.x, t = blockIdx.y;
  const int64_t lo = g * chunk, hi = min(V, lo + chunk);
  const float4 r = gate_range(logits + t * V, lo, hi);
  if (threadIdx.x == 0) parts[t * gridDim.x + g] = r;
}

__global__ __launch_bounds__(64) void gate_merge_kernel(const float4* __restrict__ parts, int G, float tau,
                                                        float delta, uint8_t* __restrict__ flags,
                                                        float* __restrict__ stats) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const bool have = lane < G;
  const float4 p = have ? parts[t * G + lane] : make_float4(-INFINITY, -INFINITY, 0.0f, 0.0f);
  float M1 = p.x, M2 = p.y;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) top2_merge(M1, M2, __shfl_xor(M1, o, 64), __shfl_xor(M2, o, 64));
  const float sc = have ? expf(p.x - M1) : 0.0f;
  const float Z = wave_sum(have ? p.z * sc : 0.0f);
  const float W = wave_sum(have ? sc * fmaf(p.x - M1, p.z, p.w) : 0.0f);
  if (lane == 0) gate_finish(M1, M2, Z, W, tau, delta, flags, stats, t);
}

// Ranges per token for a split gate: about 512 workgroups in all, at most
// 64 per token (one merge lane each), each range a multiple of 8 elements.
static void gate_split(int64_t B, int64_t V, int64_t& G, int64_t& chunk) {
  G = std::min<int64_t>(64, std::max<int64_t>(1, (512 + B - 1) / B));
  chunk = ((V + G - 1) / G + 7) / 8 * 8;
  G = (V + chunk - 1) / chunk;
}

// Scratch of the allocation-free gate entry point: the per-range partial
// statistics of gate_part_kernel (at most 16 rows x 64 ranges of float4).
// Each device holds its own copy; host code uses the per-device address
// from hipGetSymbolAddress, never the symbol itself.
constexpr size_t kGateScratchBytes = 16 * 64 * sizeof(float4);
static __device__ __align__(256) uint8_t scratch[kGateScratchBytes];

hipError_t gate_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kGateScratchBytes;
  return hipSuccess;
}

size_t gate_workspace_bytes(int64_t B, int64_t V) {
  if (B < 1 || V < 2) return 0;
  int64_t G, chunk;
  gate_split(B, V, G, chunk);
  return G > 1 ? (size_t)(B * G) * sizeof(float4) : 0;
}

hipError_t launch_gate(const uint16_t* logits, int64_t B, int64_t V, float tau, float delta, uint8_t* flags,
                       float* stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  const size_t need = gate_workspace_bytes(B, V);
  if (need == 0 || ws == nullptr || ws_bytes < need) {
    gate_kernel<<<(unsigned)B, 256, 0, stream>>>(logits, V, tau, delta, flags, stats);
    return hipGetLastError();
  }
  int64_t G, chunk;
  gate_split(B, V, G, chunk);
  float4* parts = static_cast<float4*>(ws);
  gate_part_kernel<<<dim3((unsigned)G, (unsigned)B), 256, 0, stream>>>(logits, V, chunk, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gate_merge_kernel<<<(unsigned)B, 64, 0, stream>>>(parts, (int)G, tau, delta, flags, stats);
  return hipGetLastError();
}

// -------------------------------------------------------------- KV tiles --
// 16 threads per 128-element tile, 8 elements each; amax over the 16 lanes
// by xor-shuffles; float32 scale amax / 448 and float32 division (correctly
// rounded, as the listing's division is).
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
  // clipped quotients -> E4M3FN by the hardware conversion (round to
  // nearest even, subnormals included; nothing left to saturate), two per
  // instruction, element i in byte i
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(v[i] / scale, -448.0f), 448.0f);
  uint32_t c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  c0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)c0, true);
  uint32_t c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  c1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], (int)c1, true);
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
