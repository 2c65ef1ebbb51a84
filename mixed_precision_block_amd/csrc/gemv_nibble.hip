// Decode GEMV on 8-bit weights read through their top nibble, with 8-bit
// recompute of flagged tokens (Escalating Weight Precision Only When
// Decoding Becomes Uncertain, setup paragraph).  VALU only: no MFMA.
//
// Storage (made by pack_planes_kernel): two nibble planes, hi = w >> 4
// (two's complement) and lo = w & 15, tiled by 64 rows so that a wave's
// 64 lanes read 64 consecutive 16-byte chunks (one 32-element block of 64
// rows = 1 KiB, fully coalesced).  Inside a chunk, dword q holds the
// nibbles of k = 8q + 2j in bits 4j+3..4j and of k + 1 in bits 4j+19..4j+16.
// Two masks per dword move every nibble to the top of a byte (the signed
// byte is then 16 * hi, or with lo merged in, the int8 weight); one
// sub-dword conversion per element and one pack per pair give the exact
// BF16 pair (w_k, w_{k+1}) that v_dot2_f32_bf16 multiplies with the token
// pair (x_k, x_{k+1}) -- a plain aligned dword of the BF16 row.
//
// Work split: a workgroup owns 64 rows; its four waves take interleaved
// 32-blocks of K; per block each lane turns its 16 bytes into 16 exact BF16
// pairs once and reuses them for every token (low pass: the block's x for
// all tokens is four 256-byte loads per wave that DPP row broadcasts hand
// to the dot products, with no LDS traffic; escalation: the few flagged
// tokens' x are copied to LDS by the workgroup where they fit, else come
// through the scalar cache, the address being wave-uniform).  FP32 block partials are scaled by
// the block's FP16 scale and accumulated; the four waves' sums are added in
// a fixed order through LDS.  Shapes with few row tiles split K over
// workgroups (grid y); each writes its FP32 partial sums to the caller's
// workspace and bumps its tile's arrival counter, and the last workgroup
// of a tile to arrive adds the partials in slice order, writes the output
// and resets the counter -- one launch, deterministic, no reduce kernel.
//
// Carry: the low pass can also keep its FP32 sums in a caller buffer.  As
// w = 16 hi + lo, an escalation that starts from those sums needs only the
// lo plane: y = sum_b s sum_k 16 hi x + sum_b s sum_k lo x.
#include "../../include/rq.h"
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Loads through the global address space: global loads count only against
// the vector-memory counter, while a generic (flat) load also counts
// against the LDS counter, so every LDS wait would also wait for the
// weight prefetch in flight.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const uint4* p, size_t i) {
  const u32x4 v = ((const __attribute__((address_space(1))) u32x4*)(const void*)p)[i];
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t gload2(const uint16_t* p, size_t i) {
  return ((const __attribute__((address_space(1))) uint16_t*)(const void*)p)[i];
}
__device__ __forceinline__ float f16_to_f32(uint16_t s) { return (float)__builtin_bit_cast(_Float16, s); }

// float of the signed byte N of e: one sub-dword (SDWA) conversion with
// sign extension.
template <int N>
__device__ __forceinline__ float sbyte_f32(uint32_t e) {
  float r;
  if constexpr (N == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(e));
  else if constexpr (N == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(e));
  else if constexpr (N == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(e));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(e));
  return r;
}
// Two small exact values -> BF16 pair (the conversion is exact).
__device__ __forceinline__ bf16x2 pk(float a, float b) { return (bf16x2){(__bf16)a, (__bf16)b}; }

// Nibble position p of a dword (bits 4p..4p+3) is k = 8q + 2p for p < 4
// and k = 8q + 2(p - 4) + 1 for p >= 4.  Byte n of e0 holds position 2n,
// byte n of e1 position 2n + 1, as signed bytes: pair j = (k = 8q + 2j,
// k + 1) is (e0 byte 0, e0 byte 2) for j = 0, (e1 0, e1 2) for j = 1,
// (e0 1, e0 3) for j = 2 and (e1 1, e1 3) for j = 3.
__device__ __forceinline__ void pairs_from_bytes(uint32_t e0, uint32_t e1, bf16x2* wp) {
  wp[0] = pk(sbyte_f32<0>(e0), sbyte_f32<2>(e0));
  wp[1] = pk(sbyte_f32<0>(e1), sbyte_f32<2>(e1));
  wp[2] = pk(sbyte_f32<1>(e0), sbyte_f32<3>(e0));
  wp[3] = pk(sbyte_f32<1>(e1), sbyte_f32<3>(e1));
}

// 16 * hi for the 16 pairs of a hi-plane chunk: moving each nibble to the
// top of its byte makes the signed byte 16 * hi.
__device__ __forceinline__ void unpack_hi16(const uint4 d, bf16x2 wp[16]) {
  const uint32_t dq[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) pairs_from_bytes((dq[q] << 4) & 0xF0F0F0F0u, dq[q] & 0xF0F0F0F0u, wp + 4 * q);
}

// lo (0..15) for the 16 pairs of a lo-plane chunk: each nibble in the low
// half of its byte.
__device__ __forceinline__ void unpack_lo16(const uint4 d, bf16x2 wp[16]) {
  const uint32_t dq[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) pairs_from_bytes(dq[q] & 0x0F0F0F0Fu, (dq[q] >> 4) & 0x0F0F0F0Fu, wp + 4 * q);
}

// Full 8-bit weights: byte (hi << 4 | lo) of a nibble position is the
// int8 weight.
__device__ __forceinline__ void unpack_full(const uint4 dh, const uint4 dl, bf16x2 wp[16]) {
  const uint32_t h[4] = {dh.x, dh.y, dh.z, dh.w};
  const uint32_t l[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    pairs_from_bytes(((h[q] << 4) & 0xF0F0F0F0u) | (l[q] & 0x0F0F0F0Fu),
                     (h[q] & 0xF0F0F0F0u) | ((l[q] >> 4) & 0x0F0F0F0Fu), wp + 4 * q);
}

// Planes a pass reads: the low pass the hi plane; the escalation both, or
// only lo when it starts from the low pass's FP32 carry.
enum Planes { kHi = 0, kHiLo = 1, kLo = 2 };

// Both passes share one shape of loop: a workgroup owns 64 rows and the
// K-blocks [b0, b1) of its slice (grid y splits K when there are too few
// row tiles to fill the chip); wave w takes blocks b0 + w, b0 + w + 4, ...
// The workgroup computes TB accumulator slots; slot t is token tok[t] for
// t < nt.  The four waves' sums meet in LDS in a fixed order; with one
// slice the workgroup writes BF16 outputs (the low pass: also the FP32
// carry yf when given; the escalation from the carry: adds it first),
// otherwise FP32 partials to ws[tile][slice][token][row] (16 token rows
// per slice) that the tile's last workgroup adds in slice order
// (split_finish).  gemv_tile is the escalation's loop, low_tile the low
// pass's.
constexpr int kWsTokens = 16;
constexpr int kMaxSlices = 16;  // K slices of a split launch, at most
// Arrival counters sit one per 128-byte line (32 uint32 apart): atomics of
// many tiles on one line serialize at the memory side, which made a
// 64-tile, 16-slice launch 2.5 times as long as with a line per counter.
constexpr int kCounterStride = 32;

// LDS budget for staging the flagged tokens' x in the escalation: up to
// kXStageElems elements per token of a workgroup's K range.
constexpr int kXStageElems = 4096;

// Stage x[tok[t]][32 b0, 32 b1) for t < nt into xst (4 (b1 - b0) 16-byte
// chunks per token).  Every thread of the workgroup calls it.
__device__ __forceinline__ void stage_x(uint4* xst, const uint16_t* __restrict__ x, int K, const int* tok, int nt,
                                        int b0, int b1) {
  const int kc = (b1 - b0) * 4;
  for (int i = threadIdx.x; i < nt * kc; i += 256) {
    const int t = i / kc, c = i - t * kc;
    xst[t * kc + c] = gload16(reinterpret_cast<const uint4*>(x + (size_t)tok[t] * K + (size_t)b0 * 32), c);
  }
  __syncthreads();
}

template <int TB, int kP>
__device__ __forceinline__ void gemv_tile(const uint16_t* __restrict__ x, int B, int K, int N,
                                          const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
                                          const uint16_t* __restrict__ sc, const int* tok, int nt,
                                          uint16_t* __restrict__ y, float* __restrict__ yf, float* ws,
                                          float (*red)[TB][64], uint4* xs, bool stage, int tile, int slice,
                                          int nslice) {
  static_assert(kP != kHi, "the low pass runs in low_tile");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = K >> 5;
  const int per = (nb + nslice - 1) / nslice;
  const int b0 = slice * per, b1 = min(nb, b0 + per);
  const size_t tbase = (size_t)tile * nb * 64 + lane;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + tbase;
  const uint4* lp = reinterpret_cast<const uint4*>(lo) + tbase;
  const uint16_t* sp = sc + tbase;
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;

  int b = b0 + wave;
  // the next block's planes and scale load one block ahead
  uint4 nh = make_uint4(0, 0, 0, 0), nl = make_uint4(0, 0, 0, 0);
  uint16_t ns = 0;
  if (b < b1) {
    if constexpr (kP == kHiLo) nh = gload16(hp, (size_t)b * 64);
    nl = gload16(lp, (size_t)b * 64);
    ns = gload2(sp, (size_t)b * 64);
  }
  // the copy of the flagged tokens' x to LDS overlaps the first planes' loads
  if (stage) stage_x(xs, x, K, tok, nt, b0, b1);
  for (; b < b1; b += 4) {
    const uint4 dh = nh, dl = nl;
    const float s = f16_to_f32(ns);
    {
      const int bn = b + 4 < b1 ? b + 4 : b;  // the last block reloads itself
      if constexpr (kP == kHiLo) nh = gload16(hp, (size_t)bn * 64);
      nl = gload16(lp, (size_t)bn * 64);
      ns = gload2(sp, (size_t)bn * 64);
    }
    bf16x2 wp[16];
    if constexpr (kP == kHiLo)
      unpack_full(dh, dl, wp);
    else
      unpack_lo16(dl, wp);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t >= nt) continue;  // wave-uniform
      uint32_t xq[16];
      if (xs != nullptr) {
        // the flagged tokens' x of this slice, staged in LDS by the workgroup
        const int kc = (b1 - b0) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xs[t * kc + (b - b0) * 4 + i];
          xq[4 * i] = v.x, xq[4 * i + 1] = v.y, xq[4 * i + 2] = v.z, xq[4 * i + 3] = v.w;
        }
      } else {
        // the few flagged tokens: x straight through the scalar cache
        const uint32_t* xt = reinterpret_cast<const uint32_t*>(x) + ((size_t)tok[t] * K + 32 * (size_t)b) / 2;
#pragma unroll
        for (int p = 0; p < 16; ++p) xq[p] = xt[p];
      }
      float blk = 0.0f;
#pragma unroll
      for (int p = 0; p < 16; ++p) blk = __builtin_amdgcn_fdot2_f32_bf16(wp[p], as_bf16x2(xq[p]), blk, false);
      acc[t] = fmaf(blk, s, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int o = threadIdx.x; o < TB * 64; o += 256) {
    const int t = o >> 6, l = o & 63;
    const int n = tile * 64 + l;
    if (t >= nt) continue;
    float v = ((red[0][t][l] + red[1][t][l]) + red[2][t][l]) + red[3][t][l];
    if (nslice == 1) {
      if (n < N) {
        const size_t o = (size_t)tok[t] * N + n;
        if constexpr (kP == kLo) v = yf[o] + v;
        y[o] = (uint16_t)f32_to_bf16(v);
      }
    } else {
      // coherent at device scope (visible to workgroups on other XCDs)
      __hip_atomic_store(ws + (((size_t)tile * nslice + slice) * kWsTokens + tok[t]) * 64 + l, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Split K: after a workgroup has stored its partial sums of tile `tile`
// (for the tokens in tmask), it bumps the tile's arrival counter; the last
// of the nslice workgroups to arrive adds the partials in slice order
// (kLo: onto the carry yf; kHi with yf: also storing the FP32 sums), writes
// the BF16 outputs and resets the counter to zero for the next call.
// Partials and counter are device-scope atomic accesses, coherent across
// the XCDs' separate L2s without cache-wide write-back or invalidation:
// each workgroup waits until its partial stores are complete before the
// counter is bumped, so the last arriver's device-scope loads see every
// slice.  Every thread of the workgroup calls it; nothing waits on another
// workgroup.
template <int kP>
__device__ __forceinline__ void split_finish(const float* __restrict__ ws, uint32_t* __restrict__ counters, int tile,
                                             int nslice, int N, uint32_t tmask, uint16_t* __restrict__ y,
                                             float* __restrict__ yf) {
  __shared__ uint32_t last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counters + (size_t)tile * kCounterStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last = old == (uint32_t)nslice - 1u ? 1u : 0u;
  }
  __syncthreads();
  if (!last) return;
  // every partial this thread adds is loaded first (the loads overlap; a
  // slot past the tile's slices reloads the last slice, always in bounds),
  // then each output sums its slices in order
  constexpr int kPer = kWsTokens * 64 / 256;  // outputs per thread
  float part[kPer][kMaxSlices];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int o = threadIdx.x + 256 * j, t = o >> 6, l = o & 63;
#pragma unroll
    for (int sl = 0; sl < kMaxSlices; ++sl) {
      const int sc = sl < nslice ? sl : nslice - 1;
      part[j][sl] = __hip_atomic_load(ws + (((size_t)tile * nslice + sc) * kWsTokens + t) * 64 + l,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int o = threadIdx.x + 256 * j, t = o >> 6, l = o & 63;
    const int n = tile * 64 + l;
    if (!((tmask >> t) & 1u) || n >= N) continue;
    const size_t i = (size_t)t * N + n;
    float v = kP == kLo ? yf[i] : 0.0f;
#pragma unroll
    for (int sl = 0; sl < kMaxSlices; ++sl)
      if (sl < nslice) v += part[j][sl];
    if (kP == kHi && yf != nullptr) yf[i] = v;
    y[i] = (uint16_t)f32_to_bf16(v);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(counters + (size_t)tile * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The low pass's x goes straight to registers, with no LDS traffic.  For a
// K-block, lane l (n = l % 16, its place in its row of 16 lanes) holds in
// register j of group g dword 4 (n % 4) + j of the 64-byte block of slot
// 4 g + n / 4; the wave's four rows hold the same (each group is one
// 256-byte read).  Dword p of slot 4 g + q is then register p % 4 of group
// g at lane 4 q + p / 4 of every row, and a DPP row broadcast
// (row_newbcast) hands it to all 16 lanes of the row as the dot product's
// first operand.
//
// blk[q] + sum_p w[p] . (x_2p, x_2p+1) of slot 4 g + q for q < 4, each in
// p order (the escalation's order).  A DPP instruction must not read a VGPR
// that one of the two instructions before it wrote -- its accumulator
// included -- so the four slots' dot products alternate (three others
// between two writes of one sum) and an s_nop covers the instructions
// before the block.
__device__ __forceinline__ void dot4_block_bcast(float (&blk)[4], const uint4 xg, const uint32_t (&w)[16]) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %4, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %4, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %4, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %5, %9 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %5, %9 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %5, %9 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %6, %10 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %6, %10 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %10 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %6, %10 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %7, %11 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %7, %11 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %7, %11 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %11 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %12 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %4, %12 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %4, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %4, %12 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %5, %13 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %5, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %5, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %6, %14 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %6, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %6, %14 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %7, %15 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %7, %15 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %7, %15 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %15 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %16 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %4, %16 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %4, %16 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %4, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %5, %17 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %17 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %5, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %5, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %6, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %6, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %6, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %7, %19 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %7, %19 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %7, %19 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %20 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %4, %20 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %4, %20 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %5, %21 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %21 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %5, %21 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %5, %21 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %6, %22 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %6, %22 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %22 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %6, %22 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %7, %23 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %7, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %7, %23 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "+v"(blk[0]), "+v"(blk[1]), "+v"(blk[2]), "+v"(blk[3])
      : "v"(xg.x), "v"(xg.y), "v"(xg.z), "v"(xg.w), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]),
        "v"(w[5]), "v"(w[6]), "v"(w[7]), "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]),
        "v"(w[14]), "v"(w[15]));
}

// Low pass of one 64-row tile over the K-blocks of its slice: wave w takes
// blocks b0 + w, b0 + w + 4, ...; every block's planes, scale and x load one
// block ahead.  With one slice the workgroup writes BF16 outputs (and the
// FP32 carry yf when given), otherwise FP32 partials that split_finish adds.
template <int TB>
__device__ __forceinline__ void low_tile(const uint16_t* __restrict__ x, int B, int K, int N,
                                         const uint8_t* __restrict__ hi, const uint16_t* __restrict__ sc, int nt,
                                         uint16_t* __restrict__ y, float* __restrict__ yf, float* ws,
                                         float (*red)[TB][64], int tile, int slice, int nslice) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = K >> 5;
  const int per = (nb + nslice - 1) / nslice;
  const int b0 = slice * per, b1 = min(nb, b0 + per);
  const size_t base = (size_t)tile * nb * 64 + lane;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + base;
  const uint16_t* sp = sc + base;
  constexpr int G = (TB + 3) / 4;  // groups of four slots
  const uint4* xg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int slot = 4 * g + ((lane & 15) >> 2);
    xg[g] = reinterpret_cast<const uint4*>(x + (size_t)(slot < B ? slot : B - 1) * K) + (lane & 3);
  }
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
  // Two register sets alternate (block b in one while b + 4 loads into the
  // other), so no loaded value is copied; a block past the slice's end
  // reloads the last one, always in bounds.
  auto load = [&](int blk_i, uint4 (&xr)[G], uint4& h, uint16_t& sv) {
    h = gload16(hp, (size_t)blk_i * 64), sv = gload2(sp, (size_t)blk_i * 64);
#pragma unroll
    for (int g = 0; g < G; ++g) xr[g] = gload16(xg[g], (size_t)blk_i * 4);
  };
  auto block = [&](const uint4 (&xr)[G], const uint4 h, const uint16_t sv) {
    const float s = f16_to_f32(sv);
    bf16x2 wp[16];
    unpack_hi16(h, wp);
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) w[p] = __builtin_bit_cast(uint32_t, wp[p]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float blk[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      dot4_block_bcast(blk, xr[g], w);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * g + q < TB) acc[4 * g + q] = fmaf(blk[q], s, acc[4 * g + q]);
    }
  };
  int b = b0 + wave;
  if (b < b1) {
    uint4 xa[G], xb[G], ha, hb;
    uint16_t sa, sb;
    load(b, xa, ha, sa);
    for (;;) {
      load(b + 4 < b1 ? b + 4 : b, xb, hb, sb);
      block(xa, ha, sa);
      b += 4;
      if (b >= b1) break;
      load(b + 4 < b1 ? b + 4 : b, xa, ha, sa);
      block(xb, hb, sb);
      b += 4;
      if (b >= b1) break;
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int o = threadIdx.x; o < TB * 64; o += 256) {
    const int t = o >> 6, l = o & 63;
    const int n = tile * 64 + l;
    if (t >= nt) continue;
    const float v = ((red[0][t][l] + red[1][t][l]) + red[2][t][l]) + red[3][t][l];
    if (nslice == 1) {
      if (n < N) {
        const size_t i = (size_t)t * N + n;
        if (yf != nullptr) yf[i] = v;
        y[i] = (uint16_t)f32_to_bf16(v);
      }
    } else {
      __hip_atomic_store(ws + (((size_t)tile * nslice + slice) * kWsTokens + t) * 64 + l, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int TB>
__global__ __launch_bounds__(256) void gemv_low_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                       const uint8_t* __restrict__ hi,
                                                       const uint16_t* __restrict__ sc, uint16_t* __restrict__ y,
                                                       float* __restrict__ yf, float* __restrict__ ws,
                                                       uint32_t* __restrict__ counters) {
  __shared__ float red[4][TB][64];
  low_tile<TB>(x, B, K, N, hi, sc, B < TB ? B : TB, y, yf, ws, red, blockIdx.x, blockIdx.y, gridDim.y);
  if (gridDim.y > 1) split_finish<kHi>(ws, counters, blockIdx.x, gridDim.y, N, (1u << B) - 1u, y, yf);
}

// Escalation: a workgroup takes the flagged tokens in groups of four (in
// token order), one group after another; with none flagged it exits.
constexpr int kEscTokens = 4;

// Bit t set for each flagged token t < B (wave-uniform).
__device__ __forceinline__ uint32_t flag_mask(const uint8_t* __restrict__ flags, int B) {
  uint32_t fmask = 0;
  for (int t = 0; t < B; ++t) fmask |= (flags[t] != 0 ? 1u : 0u) << t;
  return __builtin_amdgcn_readfirstlane(fmask);
}

// Takes the next (up to) four flagged tokens off fmask into tok; returns
// their count, 0 when none is left.
__device__ __forceinline__ int next_group(uint32_t& fmask, int tok[kEscTokens]) {
  int nt = 0;
#pragma unroll
  for (int t = 0; t < kEscTokens; ++t) {
    tok[t] = fmask ? __builtin_ctz(fmask) : 0;
    nt += fmask ? 1 : 0;
    fmask &= fmask - 1u;
  }
  return nt;
}

// Escalation of one 64-row tile by one wave (lane = row), over all of K.
// The sum is kept as four partials over the blocks b = w mod 4, combined
// as ((p0 + p1) + p2) + p3 -- the order of the four-wave tile (gemv_tile
// with one slice) -- so both give the same bits.  The planes of the next
// two blocks are in flight; x comes through the scalar cache (a workgroup
// copy of x in LDS made this kernel slower: every workgroup of its single
// round then waits for the copy before streaming weights).  kP is kHiLo,
// or kLo starting from the carry yf.
template <int kP>
__device__ __forceinline__ void escalate_wave_tile(const uint16_t* __restrict__ x, int K, int N,
                                                   const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
                                                   const uint16_t* __restrict__ sc, const int* tok, int nt,
                                                   uint16_t* __restrict__ y, const float* __restrict__ yf,
                                                   int tile) {
  constexpr int PF = 2;
  const int lane = threadIdx.x & 63;
  const int nb = K >> 5;
  const size_t tbase = (size_t)tile * nb * 64 + lane;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + tbase;
  const uint4* lp = reinterpret_cast<const uint4*>(lo) + tbase;
  const uint16_t* sp = sc + tbase;
  float acc[4][kEscTokens];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int t = 0; t < kEscTokens; ++t) acc[w][t] = 0.0f;
  uint4 ph[PF], pl[PF];
  uint16_t ps[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int bb = f < nb ? f : nb - 1;
    ph[f] = make_uint4(0, 0, 0, 0);
    if constexpr (kP != kLo) ph[f] = gload16(hp, (size_t)bb * 64);  // kLo: w_hi may be NULL
    pl[f] = gload16(lp, (size_t)bb * 64), ps[f] = gload2(sp, (size_t)bb * 64);
  }
  // four blocks per turn so that the partial index is static
  for (int b4 = 0; b4 < nb; b4 += 4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int b = b4 + w;
      if (b >= nb) break;
      const uint4 dh = ph[0], dl = pl[0];
      const float s = f16_to_f32(ps[0]);
#pragma unroll
      for (int f = 0; f + 1 < PF; ++f) ph[f] = ph[f + 1], pl[f] = pl[f + 1], ps[f] = ps[f + 1];
      const int bn = b + PF < nb ? b + PF : b;  // the last blocks reload themselves
      if constexpr (kP != kLo) ph[PF - 1] = gload16(hp, (size_t)bn * 64);
      pl[PF - 1] = gload16(lp, (size_t)bn * 64), ps[PF - 1] = gload2(sp, (size_t)bn * 64);
      bf16x2 wp[16];
      if constexpr (kP == kLo)
        unpack_lo16(dl, wp);
      else
        unpack_full(dh, dl, wp);
#pragma unroll
      for (int t = 0; t < kEscTokens; ++t) {
        if (t >= nt) continue;
        const uint32_t* xt = reinterpret_cast<const uint32_t*>(x) + ((size_t)tok[t] * K + 32 * (size_t)b) / 2;
        float blk = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; ++p) blk = __builtin_amdgcn_fdot2_f32_bf16(wp[p], as_bf16x2(xt[p]), blk, false);
        acc[w][t] = fmaf(blk, s, acc[w][t]);
      }
    }
  }
  const int n = tile * 64 + lane;
#pragma unroll
  for (int t = 0; t < kEscTokens; ++t) {
    float v = ((acc[0][t] + acc[1][t]) + acc[2][t]) + acc[3][t];
    if (t < nt && n < N) {
      const size_t o = (size_t)tok[t] * N + n;
      if constexpr (kP == kLo) v = yf[o] + v;
      y[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// Escalation with one wave per tile (large N, unsplit): four tiles per
// workgroup, no cross-wave reduction.
template <int kP>
__global__ __launch_bounds__(256) void gemv_escalate_wave_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                                 const uint8_t* __restrict__ hi,
                                                                 const uint8_t* __restrict__ lo,
                                                                 const uint16_t* __restrict__ sc,
                                                                 const uint8_t* __restrict__ flags,
                                                                 uint16_t* __restrict__ y,
                                                                 const float* __restrict__ yf) {
  const int tile = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (tile >= (N + 63) / 64) return;
  uint32_t fmask = flag_mask(flags, B);
  int tok[kEscTokens];
  for (int nt; (nt = next_group(fmask, tok)) > 0;) escalate_wave_tile<kP>(x, K, N, hi, lo, sc, tok, nt, y, yf, tile);
}

template <int kP>
__global__ __launch_bounds__(256) void gemv_escalate_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                            const uint8_t* __restrict__ hi,
                                                            const uint8_t* __restrict__ lo,
                                                            const uint16_t* __restrict__ sc,
                                                            const uint8_t* __restrict__ flags,
                                                            uint16_t* __restrict__ y, float* __restrict__ yf,
                                                            float* __restrict__ ws, uint32_t* __restrict__ counters,
                                                            int staged) {
  extern __shared__ uint4 xst[];  // the flagged tokens' x of this slice, when staged
  __shared__ float red[4][kEscTokens][64];
  uint32_t fmask = flag_mask(flags, B);
  const uint32_t all = fmask;
  if (all == 0) return;  // nothing flagged: no weight traffic, no arrival (the counters stay zero)
  int tok[kEscTokens];
  for (int nt; (nt = next_group(fmask, tok)) > 0;) {  // nothing (more) flagged: no weight traffic
    gemv_tile<kEscTokens, kP>(x, B, K, N, hi, lo, sc, tok, nt, y, yf, ws, red, staged ? xst : nullptr, staged != 0,
                              blockIdx.x, blockIdx.y, gridDim.y);
    __syncthreads();  // the next group reuses red and xst
  }
  if (gridDim.y > 1) split_finish<kP>(ws, counters, blockIdx.x, gridDim.y, N, all, y, yf);
}

// Grouped launch: workgroup g of the grid takes 64-row tile
// g - tile_start of the problem whose [tile_start, tile_start + ceil(N/64))
// holds g (binary search over the table; every load is wave-uniform).
__device__ __forceinline__ const rq_gemv_problem* find_problem(const rq_gemv_problem* __restrict__ probs, int count,
                                                               int64_t g) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane((int)(probs[mid].tile_start <= g))) lo = mid;
    else hi = mid - 1;
  }
  return probs + lo;
}

template <int TB>
__global__ __launch_bounds__(256) void gemv_low_grouped_kernel(const rq_gemv_problem* __restrict__ probs, int count,
                                                               int B) {
  __shared__ float red[4][TB][64];
  const rq_gemv_problem* p = find_problem(probs, count, blockIdx.x);
  const int64_t tile = (int64_t)blockIdx.x - p->tile_start;
  if (tile < 0 || tile >= (p->N + 63) / 64) return;  // a total beyond the plan
  low_tile<TB>(static_cast<const uint16_t*>(p->x_bf16), B, (int)p->K, (int)p->N, p->w_hi, p->scales_tiled,
               B < TB ? B : TB, static_cast<uint16_t*>(p->y_bf16), p->y_f32, nullptr, red, (int)tile, 0, 1);
}

// LDS for the grouped escalation's copy of the flagged tokens' x: problems
// with K up to this are staged, longer ones read x through the scalar cache.
constexpr int kGroupStageElems = 2048;

__global__ __launch_bounds__(256) void gemv_escalate_grouped_kernel(const rq_gemv_problem* __restrict__ probs,
                                                                    int count, int B,
                                                                    const uint8_t* __restrict__ flags) {
  __shared__ float red[4][kEscTokens][64];
  __shared__ uint4 xst[kEscTokens * kGroupStageElems / 8];
  uint32_t fmask = flag_mask(flags, B);
  if (fmask == 0) return;
  const rq_gemv_problem* p = find_problem(probs, count, blockIdx.x);
  const int64_t tile = (int64_t)blockIdx.x - p->tile_start;
  // problems without a low plane take no escalation
  if (p->w_lo == nullptr || tile < 0 || tile >= (p->N + 63) / 64) return;
  // four waves per tile: the sweep's 7750 tiles as one wave each would be a
  // single round whose K = 3072 tiles set the end
  // with a carry, the low pass's FP32 sums plus the lo plane alone
  const uint16_t* x = static_cast<const uint16_t*>(p->x_bf16);
  const int K = (int)p->K;
  const bool staged = K <= kGroupStageElems;
  int tok[kEscTokens];
  for (int nt; (nt = next_group(fmask, tok)) > 0;) {
    uint4* xs = staged ? xst : nullptr;
    if (p->y_f32 != nullptr)
      gemv_tile<kEscTokens, kLo>(x, B, K, (int)p->N, p->w_hi, p->w_lo, p->scales_tiled, tok, nt,
                                 static_cast<uint16_t*>(p->y_bf16), p->y_f32, nullptr, red, xs, staged, (int)tile, 0,
                                 1);
    else
      gemv_tile<kEscTokens, kHiLo>(x, B, K, (int)p->N, p->w_hi, p->w_lo, p->scales_tiled, tok, nt,
                                   static_cast<uint16_t*>(p->y_bf16), nullptr, nullptr, red, xs, staged, (int)tile,
                                   0, 1);
    __syncthreads();  // the next group reuses red and xst
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

static int gemv_tb(int64_t B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

// K slices per row tile: one when the row tiles alone give 256 workgroups,
// else enough for about `target` workgroups, each keeping at least one
// block per wave, and at most kMaxSlices (the partials the last arriver of
// a tile loads at once).  Every split launch pays one cross-workgroup
// arrival, whatever its slice count, so the count trades that against each
// workgroup's share of the work: both passes aim at 1024 workgroups, the
// fastest of 128 .. 2048 for each on a decode step of the Qwen3-0.6B shapes
// in layer order once the arrival counters sit on lines of their own (with
// packed counters the escalation's best was 128).  The workspace is sized
// for the low pass's count, which the escalation's never exceeds.
constexpr int64_t kLowTarget = 1024, kEscTarget = 1024;

static int gemv_slices(int64_t N, int64_t K, int64_t target) {
  const int64_t tiles = (N + 63) / 64, nb = K / 32;
  if (tiles == 0 || tiles >= 256) return 1;
  int64_t s = (target + tiles - 1) / tiles;
  int64_t cap = nb / 4 > 1 ? nb / 4 : 1;
  if (cap > kMaxSlices) cap = kMaxSlices;
  return (int)(s < cap ? s : cap);
}

// Workspace of a split launch: 32 KiB of per-tile arrival counters, one per
// 128-byte line (a split shape has fewer than 256 row tiles; zero between
// calls, at the same place for every shape, so shapes can share a
// workspace), then the FP32 partials [tile][slice][16 tokens][64 rows].
constexpr size_t kCounterBytes = 256 * kCounterStride * sizeof(uint32_t);

size_t gemv_workspace_bytes(int64_t B, int64_t N, int64_t K) {
  (void)B;
  const int s = gemv_slices(N, K, kLowTarget);
  return s > 1 ? kCounterBytes + (size_t)s * kWsTokens * ((N + 63) / 64 * 64) * sizeof(float) : 0;
}

// The slices of a pass: split only with a workspace of the full size (the
// escalation's count never exceeds the low pass's, which sizes it).
static int slices_for(int64_t B, int64_t N, int64_t K, size_t ws_bytes, int64_t target) {
  const int s = gemv_slices(N, K, target);
  return (s > 1 && ws_bytes >= gemv_workspace_bytes(B, N, K)) ? s : 1;
}

hipError_t launch_gemv_low(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                           const uint16_t* scales, uint16_t* y, float* yf, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  const unsigned tiles = (unsigned)((N + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const int ns = slices_for(B, N, K, ws_bytes, kLowTarget);
  const dim3 grid(tiles, ns);
  const int b = (int)B, k = (int)K, n = (int)N;
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  float* w = ns > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
  switch (gemv_tb(B)) {
    case 1: gemv_low_kernel<1><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w, cnt); break;
    case 2: gemv_low_kernel<2><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w, cnt); break;
    case 4: gemv_low_kernel<4><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w, cnt); break;
    case 8: gemv_low_kernel<8><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w, cnt); break;
    default: gemv_low_kernel<16><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w, cnt); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_escalate(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                                const uint8_t* lo, const uint16_t* scales, const uint8_t* flags, uint16_t* y,
                                float* yf, void* ws, size_t ws_bytes, hipStream_t stream) {
  const unsigned tiles = (unsigned)((N + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const int ns = slices_for(B, N, K, ws_bytes, kEscTarget);
  const int b = (int)B, k = (int)K, n = (int)N;
  if (ns == 1 && tiles >= 2048) {
    // enough tiles for one wave each: no cross-wave reduction
    if (yf)
      gemv_escalate_wave_kernel<kLo><<<(tiles + 3) / 4, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y, yf);
    else
      gemv_escalate_wave_kernel<kHiLo><<<(tiles + 3) / 4, 256, 0, stream>>>(x, b, k, n, hi, lo, scales, flags, y,
                                                                             nullptr);
    return hipGetLastError();
  }
  // four waves per tile; the flagged tokens' x of the slice staged in LDS
  // when it fits the budget
  const int64_t nb = K / 32, per = (nb + ns - 1) / ns;
  const int staged = per * 32 <= kXStageElems ? 1 : 0;
  const size_t shm = staged ? (size_t)kEscTokens * per * 32 * 2 : 0;
  const dim3 grid3(tiles, ns);
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  float* w = ns > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
  if (yf)
    gemv_escalate_kernel<kLo><<<grid3, 256, shm, stream>>>(x, b, k, n, hi, lo, scales, flags, y, yf, w, cnt, staged);
  else
    gemv_escalate_kernel<kHiLo><<<grid3, 256, shm, stream>>>(x, b, k, n, hi, lo, scales, flags, y, nullptr, w, cnt,
                                                             staged);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const rq_gemv_problem* probs, int count, int64_t total_tiles, int64_t B,
                               const uint8_t* flags, int phase, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  const int b = (int)B;
  if (phase & 1) {
    switch (gemv_tb(B)) {
      case 1: gemv_low_grouped_kernel<1><<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b); break;
      case 2: gemv_low_grouped_kernel<2><<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b); break;
      case 4: gemv_low_grouped_kernel<4><<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b); break;
      case 8: gemv_low_grouped_kernel<8><<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b); break;
      default: gemv_low_grouped_kernel<16><<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phase & 2) {
    gemv_escalate_grouped_kernel<<<(unsigned)total_tiles, 256, 0, stream>>>(probs, count, b, flags);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace rq
