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
// all tokens is one coalesced 1 KiB load per wave, broadcast through LDS;
// escalation: the few flagged tokens' x are copied to LDS by the workgroup
// where they fit, else come through the scalar cache, the address being
// wave-uniform).  FP32 block partials are scaled by
// the block's FP16 scale and accumulated; the four waves' sums are added in
// a fixed order through LDS.
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

// Every pass shares one loop: a workgroup owns 64 rows and the K-blocks
// [b0, b1) of its slice (grid y splits K when there are too few row tiles
// to fill the chip); wave w takes blocks b0 + w, b0 + w + 4, ...  The
// workgroup computes TB accumulator slots; slot t is token tok[t] for
// t < nt.  The four waves' sums meet in LDS in a fixed order; with one
// slice the workgroup writes BF16 outputs (kHi: also the FP32 carry yf
// when given; kLo: adds the carry first), otherwise FP32 partials to
// ws[slice][token][row] (16 token rows per slice) that gemv_reduce_kernel
// adds in slice order.
constexpr int kWsTokens = 16;

template <int TB, int kP>
__device__ __forceinline__ void gemv_tile(const uint16_t* __restrict__ x, int B, int K, int N,
                                          const uint8_t* __restrict__ hi, const uint8_t* __restrict__ lo,
                                          const uint16_t* __restrict__ sc, const int* tok, int nt,
                                          uint16_t* __restrict__ y, float* __restrict__ yf, float* __restrict__ ws,
                                          float (*red)[TB][64], uint4* xs, int tile, int slice, int nslice) {
  constexpr bool kFull = kP != kHi;  // an escalation pass: flagged tokens only
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = K >> 5;
  const int per = (nb + nslice - 1) / nslice;
  const int b0 = slice * per, b1 = min(nb, b0 + per);
  const size_t tbase = (size_t)tile * nb * 64 + lane;
  const uint4* hp = reinterpret_cast<const uint4*>(hi) + tbase;
  const uint4* lp = reinterpret_cast<const uint4*>(lo) + tbase;
  const uint16_t* sp = sc + tbase;
  // Low pass: x of the current block for all tokens -- lane l fetches 8
  // values (16 bytes) of token l / 4 one block ahead, the wave parks them
  // in its own 1 KiB LDS slot, and every lane reads them back as broadcasts.
  const int xt_l = (lane >> 2) < B ? (lane >> 2) : B - 1;
  const uint4* xg = reinterpret_cast<const uint4*>(x + (size_t)xt_l * K) + (lane & 3);
  uint4* const xslot = xs + wave * 64;
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0f;

  int b = b0 + wave;
  uint4 xv = make_uint4(0, 0, 0, 0);
  if (!kFull && b < b1) xv = xg[(size_t)b * 4];
  // escalation (memory-bound): the next block's planes load one block ahead
  uint4 nh = make_uint4(0, 0, 0, 0), nl = make_uint4(0, 0, 0, 0);
  uint16_t ns = 0;
  if (kFull && b < b1) {
    if constexpr (kP != kLo) nh = hp[(size_t)b * 64];
    nl = lp[(size_t)b * 64];
    ns = sp[(size_t)b * 64];
  }
  for (; b < b1; b += 4) {
    uint4 dh, dl = make_uint4(0, 0, 0, 0);
    float s;
    if constexpr (kFull) {
      dh = nh, dl = nl;
      s = f16_to_f32(ns);
      const int bn = b + 4 < b1 ? b + 4 : b;  // the last block reloads itself
      if constexpr (kP != kLo) nh = hp[(size_t)bn * 64];
      nl = lp[(size_t)bn * 64];
      ns = sp[(size_t)bn * 64];
    } else {
      dh = hp[(size_t)b * 64];
      s = f16_to_f32(sp[(size_t)b * 64]);
    }
    if constexpr (!kFull) {
      // a wave's LDS accesses complete in order: this write follows the
      // reads of the previous block and precedes the reads below
      xslot[lane] = xv;
      const int bn = b + 4 < b1 ? b + 4 : b;  // next block's x (the last reloads itself)
      xv = xg[(size_t)bn * 4];
    }
    bf16x2 wp[16];
    if constexpr (kP == kHiLo)
      unpack_full(dh, dl, wp);
    else if constexpr (kP == kLo)
      unpack_lo16(dl, wp);
    else
      unpack_hi16(dh, wp);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (kFull && t >= nt) continue;  // wave-uniform; the low pass computes every slot
      uint32_t xq[16];
      if constexpr (kFull) {
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
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xslot[4 * t + i];
          xq[4 * i] = v.x, xq[4 * i + 1] = v.y, xq[4 * i + 2] = v.z, xq[4 * i + 3] = v.w;
        }
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
        if (kP == kHi && yf != nullptr) yf[o] = v;
        y[o] = (uint16_t)f32_to_bf16(v);
      }
    } else {
      ws[((size_t)slice * kWsTokens + tok[t]) * ((size_t)((N + 63) / 64) * 64) + n] = v;
    }
  }
}

template <int TB>
__global__ __launch_bounds__(256) void gemv_low_kernel(const uint16_t* __restrict__ x, int B, int K, int N,
                                                       const uint8_t* __restrict__ hi,
                                                       const uint16_t* __restrict__ sc, uint16_t* __restrict__ y,
                                                       float* __restrict__ yf, float* __restrict__ ws) {
  __shared__ float red[4][TB][64];
  __shared__ uint4 xs[4 * 64];
  int tok[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) tok[t] = t;
  gemv_tile<TB, kHi>(x, B, K, N, hi, nullptr, sc, tok, B < TB ? B : TB, y, yf, ws, red, xs, blockIdx.x, blockIdx.y,
                     gridDim.y);
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
    xst[t * kc + c] = reinterpret_cast<const uint4*>(x + (size_t)tok[t] * K + (size_t)b0 * 32)[c];
  }
  __syncthreads();
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
    if constexpr (kP != kLo) ph[f] = hp[(size_t)bb * 64];  // kLo: w_hi may be NULL
    pl[f] = lp[(size_t)bb * 64], ps[f] = sp[(size_t)bb * 64];
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
      if constexpr (kP != kLo) ph[PF - 1] = hp[(size_t)bn * 64];
      pl[PF - 1] = lp[(size_t)bn * 64], ps[PF - 1] = sp[(size_t)bn * 64];
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
                                                            float* __restrict__ ws, int staged) {
  extern __shared__ uint4 xst[];  // the flagged tokens' x of this slice, when staged
  __shared__ float red[4][kEscTokens][64];
  uint32_t fmask = flag_mask(flags, B);
  int tok[kEscTokens];
  for (int nt; (nt = next_group(fmask, tok)) > 0;) {  // nothing (more) flagged: no weight traffic
    uint4* xs = nullptr;
    if (staged) {
      const int nb = K >> 5, per = (nb + (int)gridDim.y - 1) / (int)gridDim.y;
      const int b0 = (int)blockIdx.y * per, b1 = min(nb, b0 + per);
      if (b0 < b1) {
        stage_x(xst, x, K, tok, nt, b0, b1);
        xs = xst;
      }
    }
    gemv_tile<kEscTokens, kP>(x, B, K, N, hi, lo, sc, tok, nt, y, yf, ws, red, xs, blockIdx.x, blockIdx.y,
                              gridDim.y);
    __syncthreads();  // the next group reuses red and xst
  }
}

// y[t][n] = BF16(sum over slices of ws[slice][t][n]) in slice order, for
// every token (flags == nullptr) or the flagged ones.  carry_in (a lo-only
// escalation) is added first; carry_out (a low pass) keeps the FP32 sum.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ ws, int nslice, int B, int N,
                                                          int Np, const uint8_t* __restrict__ flags,
                                                          const float* __restrict__ carry_in,
                                                          float* __restrict__ carry_out, uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * N) return;
  const int t = (int)(i / N), n = (int)(i - (int64_t)t * N);
  if (flags && !flags[t]) return;
  float v = carry_in ? carry_in[i] : 0.0f;
  for (int sl = 0; sl < nslice; ++sl) v += ws[((size_t)sl * kWsTokens + t) * Np + n];
  if (carry_out) carry_out[i] = v;
  y[i] = (uint16_t)f32_to_bf16(v);
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
  __shared__ uint4 xs[4 * 64];
  const rq_gemv_problem* p = find_problem(probs, count, blockIdx.x);
  const int64_t tile = (int64_t)blockIdx.x - p->tile_start;
  if (tile < 0 || tile >= (p->N + 63) / 64) return;  // a total beyond the plan
  int tok[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) tok[t] = t;
  gemv_tile<TB, kHi>(static_cast<const uint16_t*>(p->x_bf16), B, (int)p->K, (int)p->N, p->w_hi, nullptr,
                     p->scales_tiled, tok, B < TB ? B : TB, static_cast<uint16_t*>(p->y_bf16), p->y_f32, nullptr,
                     red, xs, (int)tile, 0, 1);
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
    if (staged) stage_x(xst, x, K, tok, nt, 0, K >> 5);
    uint4* xs = staged ? xst : nullptr;
    if (p->y_f32 != nullptr)
      gemv_tile<kEscTokens, kLo>(x, B, K, (int)p->N, p->w_hi, p->w_lo, p->scales_tiled, tok, nt,
                                 static_cast<uint16_t*>(p->y_bf16), p->y_f32, nullptr, red, xs, (int)tile, 0, 1);
    else
      gemv_tile<kEscTokens, kHiLo>(x, B, K, (int)p->N, p->w_hi, p->w_lo, p->scales_tiled, tok, nt,
                                   static_cast<uint16_t*>(p->y_bf16), nullptr, nullptr, red, xs, (int)tile, 0, 1);
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
// else enough for about 512 workgroups, each keeping at least one block
// per wave.
int gemv_slices(int64_t N, int64_t K) {
  const int64_t tiles = (N + 63) / 64, nb = K / 32;
  if (tiles == 0 || tiles >= 256) return 1;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t cap = nb / 4 > 1 ? nb / 4 : 1;
  return (int)(s < cap ? s : cap);
}

size_t gemv_workspace_bytes(int64_t B, int64_t N, int64_t K) {
  (void)B;
  const int s = gemv_slices(N, K);
  return s > 1 ? (size_t)s * kWsTokens * ((N + 63) / 64 * 64) * sizeof(float) : 0;
}

static int slices_for(int64_t B, int64_t N, int64_t K, size_t ws_bytes) {
  const int s = gemv_slices(N, K);
  return (s > 1 && ws_bytes >= gemv_workspace_bytes(B, N, K)) ? s : 1;
}

static hipError_t launch_reduce(const float* ws, int nslice, int64_t B, int64_t N, const uint8_t* flags,
                                const float* carry_in, float* carry_out, uint16_t* y, hipStream_t stream) {
  const int64_t total = B * N;
  gemv_reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
      ws, nslice, (int)B, (int)N, (int)((N + 63) / 64 * 64), flags, carry_in, carry_out, y);
  return hipGetLastError();
}

hipError_t launch_gemv_low(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                           const uint16_t* scales, uint16_t* y, float* yf, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  const unsigned tiles = (unsigned)((N + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const int ns = slices_for(B, N, K, ws_bytes);
  const dim3 grid(tiles, ns);
  const int b = (int)B, k = (int)K, n = (int)N;
  float* w = static_cast<float*>(ws);
  switch (gemv_tb(B)) {
    case 1: gemv_low_kernel<1><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w); break;
    case 2: gemv_low_kernel<2><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w); break;
    case 4: gemv_low_kernel<4><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w); break;
    case 8: gemv_low_kernel<8><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w); break;
    default: gemv_low_kernel<16><<<grid, 256, 0, stream>>>(x, b, k, n, hi, scales, y, yf, w); break;
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ns > 1) e = launch_reduce(w, ns, B, N, nullptr, nullptr, yf, y, stream);
  return e;
}

hipError_t launch_gemv_escalate(const uint16_t* x, int64_t B, int64_t K, int64_t N, const uint8_t* hi,
                                const uint8_t* lo, const uint16_t* scales, const uint8_t* flags, uint16_t* y,
                                float* yf, void* ws, size_t ws_bytes, hipStream_t stream) {
  const unsigned tiles = (unsigned)((N + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const int ns = slices_for(B, N, K, ws_bytes);
  const int b = (int)B, k = (int)K, n = (int)N;
  float* w = static_cast<float*>(ws);
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
  if (yf)
    gemv_escalate_kernel<kLo><<<grid3, 256, shm, stream>>>(x, b, k, n, hi, lo, scales, flags, y, yf, w, staged);
  else
    gemv_escalate_kernel<kHiLo><<<grid3, 256, shm, stream>>>(x, b, k, n, hi, lo, scales, flags, y, nullptr, w,
                                                             staged);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ns > 1) e = launch_reduce(w, ns, B, N, flags, yf, nullptr, y, stream);
  return e;
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
