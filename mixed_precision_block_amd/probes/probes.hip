// Hardware probes behind the ceilings quoted for the library's kernels:
// the sustained matrix-instruction rate and shader clock on constant versus
// random operand bits, how far VALU dequantization overlaps BF16 matrix
// instructions (rqp_probe), L2 and HBM streaming into LDS the way the
// pipelined GEMM loads (rqp_stream), LDS reads (rqp_lds), and the cost of
// back-to-back launches, with and without the split-K GEMV's cross-workgroup
// arrival (rqp_launch).
// Measurement only: nothing in librq calls these, and their results are
// never used as outputs of the library.
//
// Each matrix-instruction probe wave keeps eight independent accumulators and issues eight
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

namespace rqp {

// L2 -> LDS streaming as the pipelined GEMM does it: eight waves per
// workgroup (one workgroup per CU) fill a ring of NSTG LDS stages of SB
// bytes with 16-byte buffer-to-LDS loads (lane l of a load at byte 16 l of
// a 1 KiB slot), wait for the stage in flight with the GEMM's count of
// outstanding loads and meet one barrier per stage; nothing is computed.
// Workgroup g reads the window [win * (g % nwin), + win) of src (win a
// power of two), wrapping inside it; the buffer resource spans exactly
// src_bytes, so any offset beyond it reads zeros without touching memory.
template <int NSTG, int SB>
__global__ __launch_bounds__(512, 1) void stream_kernel(const uint8_t* __restrict__ src, uint32_t src_bytes,
                                                       uint32_t win, uint32_t nwin, int stages,
                                                       float* __restrict__ out, uint64_t* __restrict__ t) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTG * SB];
  constexpr int kLoads = SB / 1024 / 8;  // 1 KiB loads per wave per stage
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)src_bytes, 0x00020000);
  const uint32_t base = win * (blockIdx.x % nwin);
  auto issue = [&](int s) {
    uint8_t* st = smem + (s % NSTG) * SB;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint32_t slot = (uint32_t)(wave * kLoads + i);
      const uint32_t off = base + (((uint32_t)s * (uint32_t)SB + slot * 1024u + 16u * (uint32_t)lane) & (win - 1u));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(st + slot * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  stamp(t, 0);
  for (int s = 0; s < NSTG - 1; ++s) issue(s);
  for (int s = 0; s < stages; ++s) {
    issue(s + NSTG - 1);
    // the oldest stage in flight has landed: NSTG - 1 stages' loads may still be outstanding
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((NSTG - 1) * kLoads) : "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  stamp(t, 1);
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = (float)smem[(threadIdx.x * 16) % (NSTG * SB)];
}

// Launch latency: an empty kernel; one that reads one dword per thread; and
// one whose workgroups meet at a device-scope arrival counter the way the
// split-K GEMV finishes (each stores a partial with a device-scope store,
// waits for it, bumps the counter; the last to arrive loads every partial,
// writes the sum and resets the counter).  No workgroup waits for another.
__global__ __launch_bounds__(256) void empty_kernel() {}

__global__ __launch_bounds__(256) void touch_kernel(const float* __restrict__ x, float* __restrict__ y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  y[i] = x[i] + 1.0f;
}

constexpr unsigned kMaxArrivals = 16;  // slices of one tile, at most

// grid (tiles, slices): workgroup (t, s) stores its partial, waits for the
// store, bumps tile t's counter; the tile's last workgroup loads the
// tile's partials (all loads issued before any is added), writes their sum
// and resets the counter.
__global__ __launch_bounds__(256) void arrival_kernel(float* __restrict__ part, unsigned* __restrict__ counter,
                                                      unsigned cstride, float* __restrict__ y) {
  const unsigned tile = blockIdx.x, slices = gridDim.y;
  const size_t i = ((size_t)tile * slices + blockIdx.y) * 256 + threadIdx.x;
  __hip_atomic_store(part + i, (float)threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial store is complete
  __syncthreads();
  __shared__ unsigned last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(counter + (size_t)tile * cstride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           slices - 1;
  __syncthreads();
  if (last) {
    float v[kMaxArrivals];
#pragma unroll
    for (unsigned b = 0; b < kMaxArrivals; ++b)
      v[b] = __hip_atomic_load(part + ((size_t)tile * slices + min(b, slices - 1)) * 256 + threadIdx.x,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float s = 0.0f;
#pragma unroll
    for (unsigned b = 0; b < kMaxArrivals; ++b) s += b < slices ? v[b] : 0.0f;
    y[(size_t)tile * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0)
      __hip_atomic_store(counter + (size_t)tile * cstride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace rqp

// L2 -> LDS streaming: kind 0 two 64 KiB stages, 1 three 32 KiB stages,
// 2 four 32 KiB stages; 512-thread workgroups, one per CU.  src of
// src_bytes (< 2^31); workgroup g reads window g % nwin of win bytes
// (win a power of two of at least 1 KiB, nwin * win <= src_bytes).  out: blocks * 512
// floats; stamps: blocks * 4 u64.  Returns a hipError_t value, or 1 for a
// bad argument.
extern "C" int rqp_stream(int kind, const void* src, uint32_t src_bytes, uint32_t win, uint32_t nwin, int blocks,
                          int stages, void* out, void* stamps, hipStream_t stream) {
  if (win < 1024 || (win & (win - 1)) || nwin == 0 || (uint64_t)win * nwin > src_bytes || src_bytes >= 0x80000000u)
    return 1;
  const uint8_t* s = (const uint8_t*)src;
  float* y = (float*)out;
  uint64_t* t = (uint64_t*)stamps;
  switch (kind) {
    case 0: rqp::stream_kernel<2, 65536><<<blocks, 512, 0, stream>>>(s, src_bytes, win, nwin, stages, y, t); break;
    case 1: rqp::stream_kernel<3, 32768><<<blocks, 512, 0, stream>>>(s, src_bytes, win, nwin, stages, y, t); break;
    case 2: rqp::stream_kernel<4, 32768><<<blocks, 512, 0, stream>>>(s, src_bytes, win, nwin, stages, y, t); break;
    default: return 1;
  }
  return (int)hipGetLastError();
}

// Launch-latency kernels: kind 0 empty, 1 touch (x, y: blocks * 256
// floats), 2 arrival with blocks tiles of `slices` workgroups (slices <= 16;
// part: blocks * slices * 256 floats, counter: tile t's counter at element
// t * cstride of blocks * cstride zeroed unsigned, y: blocks * 256 floats).
// Returns a hipError_t value, or 1 for a bad kind or size.
extern "C" int rqp_launch(int kind, int blocks, int slices, int cstride, void* a, void* b, void* c,
                          hipStream_t stream) {
  if (blocks <= 0 || (kind == 2 && (slices <= 0 || slices > (int)rqp::kMaxArrivals || cstride <= 0))) return 1;
  switch (kind) {
    case 0: rqp::empty_kernel<<<blocks, 256, 0, stream>>>(); break;
    case 1: rqp::touch_kernel<<<blocks, 256, 0, stream>>>((const float*)a, (float*)b); break;
    case 2:
      rqp::arrival_kernel<<<dim3(blocks, slices), 256, 0, stream>>>((float*)a, (unsigned*)b, (unsigned)cstride,
                                                                   (float*)c);
      break;
    default: return 1;
  }
  return (int)hipGetLastError();
}

namespace rqp {

// LDS read rate: each wave of a 256-thread workgroup reads 16 bytes per lane
// (ds_read_b128, lane l at byte 16 l of its wave's 1 KiB, no bank
// conflict) eight times per iteration from a 32 KiB buffer it filled once,
// xor-folding the values so that every read is kept.
__global__ __launch_bounds__(256) void lds_read_kernel(int iters, float* __restrict__ out, uint64_t* __restrict__ t) {
  __shared__ uint4 buf[2048];  // 32 KiB
  for (int i = threadIdx.x; i < 2048; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint4 acc = make_uint4(0, 0, 0, 0);
  stamp(t, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint4 v = buf[((wave * 8 + r + it) & 31) * 64 + lane];
      acc.x ^= v.x, acc.y ^= v.y, acc.z ^= v.z, acc.w ^= v.w;
    }
  }
  stamp(t, 1);
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

}  // namespace rqp

// LDS read rate: blocks workgroups of 256 threads (blocks / 256 per CU; a
// CU holds at most 8 of them by waves per SIMD), iters iterations of eight
// 16-byte reads per lane.  out: blocks * 256 floats; stamps: blocks * 4 u64.
// Returns a hipError_t value, or 1 for a bad size.
extern "C" int rqp_lds(int blocks, int iters, void* out, void* stamps, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0) return 1;
  rqp::lds_read_kernel<<<blocks, 256, 0, stream>>>(iters, (float*)out, (uint64_t*)stamps);
  return (int)hipGetLastError();
}
