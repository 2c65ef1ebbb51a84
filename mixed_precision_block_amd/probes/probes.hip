// Hardware probes behind the ceilings quoted for the GEMM kernels: the
// sustained matrix-instruction rate and shader clock on constant versus
// random operand bits, and how far VALU dequantization overlaps BF16
// matrix instructions.  Measurement only: nothing in librq calls these,
// and their results are never used as GEMM outputs.
//
// Each probe wave keeps eight independent accumulators and issues eight
// matrix instructions per loop iteration on operands it loaded once.  Lane 0
// of every workgroup's first wave reads the shader cycle counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) before and
// after the loop, so the host can divide the two and read the shader clock
// under that load.  Every thread writes one float of its accumulators so
// that the compiler keeps the work; all accesses stay inside the buffers the
// host sizes from the grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rqp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

enum Kind { kFp4 = 0, kFp8 = 1, kBf16 = 2, kBf16Deq = 3, kDeqOnly = 4 };

__device__ __forceinline__ void stamp(uint64_t* t, int slot) {
  if (threadIdx.x == 0) {
    const uint64_t c = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    t[(size_t)blockIdx.x * 4 + 2 * slot] = c;
    t[(size_t)blockIdx.x * 4 + 2 * slot + 1] = r;
  }
}

// ops: 12 dwords per thread (operand bits); scales: one dword per thread.
template <int K>
__global__ __launch_bounds__(256, 2) void probe_kernel(const uint32_t* __restrict__ ops,
                                                       const uint32_t* __restrict__ scales, int iters,
                                                       float* __restrict__ out, uint64_t* __restrict__ t) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t c[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) c[i] = ops[tid * 12 + i];
  const uint32_t sc = scales[tid];
  v16f acc[8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][e] = 0.0f;
  v8bf bo[6];
#pragma unroll
  for (int i = 0; i < 6; ++i)
    bo[i] = __builtin_bit_cast(v8bf, (v4i){(int)c[2 * i], (int)c[2 * i + 1], (int)c[(2 * i + 2) % 12],
                                           (int)c[(2 * i + 3) % 12]});
  const float fs = __builtin_bit_cast(float, 0x3F800000u);
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
    if constexpr (K == kFp4 || K == kFp8) {
      const v8i a0 = {(int)c[0], (int)c[1], (int)c[2], (int)c[3], (int)c[4], (int)c[5], (int)c[6], (int)c[7]};
      const v8i a1 = {(int)c[4], (int)c[5], (int)c[6], (int)c[7], (int)c[8], (int)c[9], (int)c[10], (int)c[11]};
      constexpr int f = K == kFp4 ? 4 : 0;
#pragma unroll
      for (int a = 0; a < 8; ++a)
        acc[a] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a & 1 ? a1 : a0, a & 2 ? a1 : a0, acc[a], f, f, 0,
                                                                  (int)sc, 0, (int)(sc >> 8));
    } else {
      if constexpr (K == kBf16Deq || K == kDeqOnly) {
        // six 8-element BF16 operands from twelve code dwords: 24 scaled
        // FP8 -> BF16 conversions per eight matrix instructions, the ratio
        // of a 128 x 64 wave tile
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const v2bf p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[2 * i], fs, false);
          const v2bf q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[2 * i], fs, true);
          const v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[2 * i + 1], fs, false);
          const v2bf s = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[2 * i + 1], fs, true);
          bo[i] = (v8bf){p.x, p.y, q.x, q.y, r.x, r.y, s.x, s.y};
        }
        // vary the codes per iteration (finite codes stay finite)
#pragma unroll
        for (int i = 0; i < 12; ++i) c[i] ^= (uint32_t)it & 0x01010101u;
      }
      if constexpr (K == kDeqOnly) {
#pragma unroll
        for (int i = 0; i < 6; ++i) asm volatile("" ::"v"(bo[i]));
      } else {
#pragma unroll
        for (int a = 0; a < 8; ++a)
          acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[4 + (a & 1)], bo[a >> 1], acc[a], 0, 0, 0);
      }
    }
  }
  stamp(t, 1);
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[a][e];
#pragma unroll
  for (int i = 0; i < 6; ++i) s += (float)bo[i][0];
  out[tid] = s;
}

}  // namespace rqp

// kind: 0 FP4 scaled 32x32x64, 1 FP8 scaled 32x32x64, 2 BF16 32x32x16,
// 3 BF16 32x32x16 fed by 24 scaled FP8 -> BF16 conversions per eight,
// 4 the conversions alone.  ops: blocks * 256 * 12 dwords; scales:
// blocks * 256 dwords; out: blocks * 256 floats; stamps: blocks * 4 u64.
// Returns a hipError_t value (0 on success); 1 for an unknown kind.
extern "C" int rqp_probe(int kind, const void* ops, const void* scales, int blocks, int iters, void* out,
                         void* stamps, hipStream_t stream) {
  const uint32_t* o = (const uint32_t*)ops;
  const uint32_t* s = (const uint32_t*)scales;
  float* y = (float*)out;
  uint64_t* t = (uint64_t*)stamps;
  switch (kind) {
    case 0: rqp::probe_kernel<0><<<blocks, 256, 0, stream>>>(o, s, iters, y, t); break;
    case 1: rqp::probe_kernel<1><<<blocks, 256, 0, stream>>>(o, s, iters, y, t); break;
    case 2: rqp::probe_kernel<2><<<blocks, 256, 0, stream>>>(o, s, iters, y, t); break;
    case 3: rqp::probe_kernel<3><<<blocks, 256, 0, stream>>>(o, s, iters, y, t); break;
    case 4: rqp::probe_kernel<4><<<blocks, 256, 0, stream>>>(o, s, iters, y, t); break;
    default: return 1;
  }
  return (int)hipGetLastError();
}
