// Pipelined block-scaled GEMM for gfx950: Y[M x N] = A . W^T, K-major.
//
// Same contraction as gemm.hip (ARCQuant unified GEMM; Day-0 page section V
// item 3: block scales applied inside the matrix core), organized for
// throughput on large problems:
//
// * A pipeline stage holds one RB-byte chunk (RB = 128) of every row of the
//   A and W tiles: 2 RB elements of MXFP4, RB of MXFP8 or RB / 2 of BF16, so
//   each stage carries the same matrix-core work whatever the format.
//   128-byte chunks are whole cache lines for the global loads.  When K is
//   not a whole number of stages the last stage is partial: its loads run
//   past the row (into the next row, or zeros past the buffer) and only its
//   valid MFMA slices are computed.
// * Operands go straight from global memory into LDS (gfx950's 16-byte
//   buffer loads to LDS; scales by 4-byte ones), NSTG stages deep: while one
//   stage feeds the MFMAs the next NSTG - 1 are in flight.  No registers
//   hold operands on the way and no LDS writes are issued by the waves.  The
//   buffer resources span the tile's rows, so rows past M or N load zeros.
//   Each step ends with one wait on this wave's loads of the next stage and
//   one barrier.
// * LDS rows are RB bytes of 16-byte chunks, XOR-swizzled per row so that
//   the fragment reads of consecutive rows hit distinct banks (checked for
//   both 32- and 64-bank LDS models).
// * WMW x WNW waves, each owning a (BM/WMW) x (BN/WNW) quadrant of MFMA
//   tiles of 32 x 32; accumulators live in AGPRs.  With KS = 2 there are
//   two such grids, each summing every other slice of each stage, and the
//   second grid's sums are added to the first's through LDS at the end.  256 x 256 tiles use
//   eight waves (two per SIMD, so one wave's waits overlap the other's
//   MFMAs), 128 x 128 tiles four.
// * Workgroups are ordered so that consecutive tiles land on the same XCD
//   (the dispatcher deals workgroups round-robin over the 8 XCDs) and each
//   XCD's tiles form a compact block of 4 M-tiles, sharing A and W panels in
//   that XCD's L2.
//
// Operand layout per MFMA is the one pinned for gemm.hip: FP4 lane half h
// holds K [32h, 32h+32) of a 64-deep slice; FP8 lane half h holds
// K [16h, 16h+16) and [32+16h, 32+16h+16); BF16 lane half h holds 8
// elements at 8h of a 16-deep slice.  Slice kk's block scales are bytes
// 2 kk and 2 kk + 1 of the row's stage scales, lane half h taking 2 kk + h.
//
// MXFP8 (FMT 2) reads the FP8 fragments the same way but does not use the
// FP8 scaled instruction, which truncates products inside runs of 8 K
// terms: each lane dequantizes its codes with their block scale to BF16
// (exact) and the slice becomes four BF16 MFMAs with FP32 accumulation.
// FMT 4 issues the FP8 scaled instruction on the same data.
#include <type_traits>

#include "rq_block.h"
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

template <int FMT, int RB>
struct PipeTraits;
template <int RB>
struct PipeTraits<1, RB> {  // MXFP4: 2 RB K per stage in 64-deep slices
  static constexpr int kStepElems = 2 * RB, kKK = 2 * RB / 64, kCbsz = 4, kSBPR = 2 * RB / 32;
  static constexpr bool kScaled = true;
};
template <int RB>
struct PipeTraits<2, RB> {  // MXFP8: RB K per stage in 64-deep slices
  static_assert(RB == 128, "MXFP8 stages are 128 bytes (whole scale dwords)");
  static constexpr int kStepElems = RB, kKK = RB / 64, kCbsz = 0, kSBPR = RB / 32;
  static constexpr bool kScaled = true;
};
template <int RB>
struct PipeTraits<4, RB> : PipeTraits<2, RB> {};  // MXFP8 on the FP8 scaled MFMA: same stages
template <int RB>
struct PipeTraits<3, RB> {  // BF16: RB / 2 K per stage in 16-deep slices
  static constexpr int kStepElems = RB / 2, kKK = RB / 32, kCbsz = 0, kSBPR = 0;
  static constexpr bool kScaled = false;
};

// Chunk swizzle of a 128-byte LDS row r: chunk bits (r0 ^ r3, r2, r1).
template <int RB>
__device__ __forceinline__ int swz(int r) {
  static_assert(RB == 128, "128-byte stage rows");
  return ((r ^ (r >> 3)) & 1) | ((r >> 1) & 2) | ((r << 1) & 4);
}

// One wave-wide direct load into LDS: lane l's 16 (4) bytes land at
// lds + 16 l (4 l).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

template <int FMT, int BM, int BN, int RB, int WMW, int WNW, int NSTG, int KS = 1>
struct DmaCfg {
  using T = PipeTraits<FMT, RB>;
  static constexpr int NW = WMW * WNW * KS, NT = 64 * NW;  // KS groups of WMW x WNW waves
  static constexpr int TM = BM / 32 / WMW, TN = BN / 32 / WNW;
  static constexpr int WM = BM / WMW, WN = BN / WNW;
  static constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                // rows per wave-wide 16-byte DMA (1 KB)
  static constexpr int IA = BM / RPI, IW = BN / RPI;  // DMAs per stage of the A / W tile
  static constexpr int DPW = (IA + IW) / NW;          // operand DMAs per wave per stage
  static constexpr int SA = BM * RB, SW = BN * RB;
  static constexpr int SBPR = T::kSBPR;
  // Scale rows per stage: the tile's A then W rows, padded (rows past the W
  // tile read as zeros: they lie beyond its buffer range) so that the
  // 256-byte scale DMAs split evenly over the waves.
  static constexpr int SRU = SBPR > 0 ? 256 * NW / SBPR : 1;
  static constexpr int SR = SBPR > 0 ? (BM + BN + SRU - 1) / SRU * SRU : 0;
  static constexpr int SS = SR * SBPR;
  static constexpr int IS = SS / 256;                 // dword DMAs of the stage's scales (0 for BF16)
  static constexpr int SPW = IS / NW;
  static constexpr int DW = DPW + SPW;                // DMAs per wave per stage
  static constexpr int STAGE = SA + SW + SS;
  // every wave issues the same loads per stage, so the load-count waits are exact
  static_assert((IA + IW) % NW == 0 && IS % NW == 0, "loads split evenly over the waves");
  static_assert(SS % 256 == 0, "whole scale DMAs");
  static_assert((BM * SBPR) % 256 == 0, "a scale DMA stays on one side");
  static_assert(NSTG * STAGE <= 160 * 1024, "stages fit the LDS");
};

template <int FMT, int EPI, int BM, int BN, int RB, int WMW, int WNW, int NSTG, int KS>
__global__ __launch_bounds__(64 * WMW * WNW * KS, 1) void gemm_pipe_kernel(const uint8_t* __restrict__ A,
                                                                      const uint8_t* __restrict__ As,
                                                                      const uint8_t* __restrict__ W,
                                                                      const uint8_t* __restrict__ Ws, int M, int N,
                                                                      int K, void* __restrict__ Y,
                                                                      uint8_t* __restrict__ Ys, int tiles_m,
                                                                      int tiles_n) {
  using C = DmaCfg<FMT, BM, BN, RB, WMW, WNW, NSTG, KS>;
  using T = PipeTraits<FMT, RB>;
  // two K groups only for the exact MXFP8 path, whose slices reload their
  // scale dwords each time (the other formats load them every other slice)
  static_assert(KS == 1 || (KS == 2 && FMT == 2), "K groups: one, or two on the exact MXFP8 path");
  constexpr int TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTG * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // K group kg of the workgroup's KS groups takes the stage slices kk with
  // kk % KS == kg; inside a group, waves form the WMW x WNW grid
  const int kg = wave / (WMW * WNW), wg = wave % (WMW * WNW);
  const int wm = wg / WNW, wn = wg % WNW;
  const int half = lane >> 5, lrow = lane & 31;

  // XCD-aware tile order
  const int pid = blockIdx.x, nt = tiles_m * tiles_n;
  const int v = (nt % 8 == 0) ? (pid % 8) * (nt / 8) + pid / 8 : pid;
  constexpr int GM = 4;
  const int group = v / (GM * tiles_n), first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (v % (GM * tiles_n)) % gsz, tn = (v % (GM * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  constexpr bool kF8 = FMT == 2 || FMT == 4;  // E4M3 codes, one byte per element
  const uint32_t ld = FMT == 1 ? (uint32_t)K / 2 : (kF8 ? (uint32_t)K : 2u * (uint32_t)K);  // row bytes
  const uint32_t ksb = (uint32_t)K / 32;
  const int nk = (K + T::kStepElems - 1) / T::kStepElems;  // stages, the last one maybe partial
  const int nfull = K / T::kStepElems;
  const int tail_kk = (K - nfull * T::kStepElems) / (T::kStepElems / T::kKK);  // valid slices of a partial stage

  const uint32_t a_rows = (uint32_t)min(BM, M - m0), w_rows = (uint32_t)min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + (size_t)m0 * ld), 0, (int)(a_rows * ld), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)n0 * ld), 0, (int)(w_rows * ld), 0x00020000);
  __amdgpu_buffer_rsrc_t rsa = ra, rsw = rw;
  if constexpr (T::kScaled) {
    rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(As + (size_t)m0 * ksb), 0, (int)(a_rows * ksb), 0x00020000);
    rsw = __builtin_amdgcn_make_buffer_rsrc((void*)(Ws + (size_t)n0 * ksb), 0, (int)(w_rows * ksb), 0x00020000);
  }

  // Direct global-to-LDS loads: each wave-wide 16-byte load fills 1 KB of
  // LDS, lane l at byte 16 l, i.e. RPI whole rows.  The swizzle is applied
  // on the global side: the lane writing physical chunk p of row r reads
  // logical chunk p ^ swz(r).
  uint32_t voff[C::DPW];
#pragma unroll
  for (int i = 0; i < C::DPW; ++i) {
    const int q = wave * C::DPW + i;
    const int r = (q < C::IA ? q : q - C::IA) * C::RPI + lane / C::CPR;
    voff[i] = (uint32_t)r * ld + 16u * (uint32_t)((lane % C::CPR) ^ swz<RB>(r));
  }
  uint32_t soff[C::SPW > 0 ? C::SPW : 1];
  if constexpr (T::kScaled) {
#pragma unroll
    for (int i = 0; i < C::SPW; ++i) {
      const int q = wave * C::SPW + i;
      const int rho = (q * 256 + 4 * lane) / C::SBPR;  // scale row (A rows, then W rows)
      const int b = (4 * lane) % C::SBPR;
      soff[i] = (uint32_t)(rho < BM ? rho : rho - BM) * ksb + (uint32_t)b;
    }
  }

  // Stages past the end read at an offset beyond every buffer range (zeros,
  // no memory access), so every step issues the same number of loads and
  // the load-count waits below stay exact.
  constexpr uint32_t kPastEnd = 0x80000000u;
  auto issue = [&](uint8_t* st, int s) {
    const uint32_t kb = s < nk ? (uint32_t)s * RB : kPastEnd;
#pragma unroll
    for (int i = 0; i < C::DPW; ++i) {
      const int q = wave * C::DPW + i;
      const bool is_a = q < C::IA;
      uint8_t* dst = st + (is_a ? q * 1024 : C::SA + (q - C::IA) * 1024);
      load_lds16(is_a ? ra : rw, dst, voff[i] + kb);
    }
    if constexpr (T::kScaled) {
      const uint32_t sk = s < nk ? (uint32_t)s * C::SBPR : kPastEnd;
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const int q = wave * C::SPW + i;
        const bool is_a = q * 256 < BM * C::SBPR;
        uint8_t* dst = st + C::SA + C::SW + q * 256;
        load_lds4(is_a ? rsa : rsw, dst, soff[i] + sk);
      }
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // A stage in slices of 64 K (16 K for BF16): each slice's fragments are
  // read from LDS, then its MFMAs issue (the compiler interleaves the next
  // slice's reads with them).  Each row's scales come as one dword per two
  // slices; the lane's byte is extracted per slice.
  auto compute = [&](const uint8_t* st, int nkk) {
    constexpr int KK = T::kKK;
    constexpr int NQ = kF8 ? 2 : 1;  // 16-byte chunks per lane per fragment
    const uint8_t* sc = st + C::SA + C::SW;
    int za[TM], zb[TN];
    // the row's scale dword holding slices kk of the current pair
    uint32_t sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) za[i] = swz<RB>(wm * C::WM + i * 32 + lrow);
#pragma unroll
    for (int j = 0; j < TN; ++j) zb[j] = swz<RB>(wn * C::WN + j * 32 + lrow);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk >= nkk) break;  // nkk == KK (folded) except in a partial last stage
      if (KS > 1 && kk % KS != kg) continue;
      v4i fa[TM][NQ], fb[TN][NQ];
      // 16-byte chunk(s) of this slice for the lane's half
      const int c0 = kF8 ? kk * 4 + half : kk * 2 + half;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* row = st + (wm * C::WM + i * 32 + lrow) * RB;
        fa[i][0] = *reinterpret_cast<const v4i*>(row + 16 * (c0 ^ za[i]));
        if constexpr (NQ == 2) fa[i][1] = *reinterpret_cast<const v4i*>(row + 16 * ((c0 + 2) ^ za[i]));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* row = st + C::SA + (wn * C::WN + j * 32 + lrow) * RB;
        fb[j][0] = *reinterpret_cast<const v4i*>(row + 16 * (c0 ^ zb[j]));
        if constexpr (NQ == 2) fb[j][1] = *reinterpret_cast<const v4i*>(row + 16 * ((c0 + 2) ^ zb[j]));
      }
      // scale byte 2 kk + half of the row's stage scales: dword kk / 2
      const int sbyte = 2 * kk + half;
      uint32_t esa[TM], esb[TN];
      if constexpr (FMT == 2) {
        // exact MXFP8: both block scales of the slice, as floats; each lane
        // dequantizes its codes to BF16 and the BF16 MFMA accumulates in FP32
        if (KS > 1 || kk % 2 == 0) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
            sa[i] = *reinterpret_cast<const uint32_t*>(sc + (wm * C::WM + i * 32 + lrow) * C::SBPR + 4 * (kk / 2));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            sb[j] = *reinterpret_cast<const uint32_t*>(sc + (BM + wn * C::WN + j * 32 + lrow) * C::SBPR +
                                                       4 * (kk / 2));
        }
        // MFMA q of the slice takes 8 codes per lane: dwords 2 (q % 2), +1
        // of chunk q / 2 (lane half h: K 16 h + 8 (q % 2) of block q / 2),
        // the same K for both operands, so the four MFMAs cover the slice
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sh = 8 * ((2 * kk + q / 2) & 3);
          rq_v8bf da[TM], dw[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const v4i c = fa[i][q / 2];
            const float f = e8m0_to_f32(__builtin_amdgcn_ubfe(sa[i], sh, 8));
            da[i] = q % 2 ? deq8_e4m3(c.z, c.w, f) : deq8_e4m3(c.x, c.y, f);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const v4i c = fb[j][q / 2];
            const float f = e8m0_to_f32(__builtin_amdgcn_ubfe(sb[j], sh, 8));
            dw[j] = q % 2 ? deq8_e4m3(c.z, c.w, f) : deq8_e4m3(c.x, c.y, f);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dw[j], da[i], acc[i][j], 0, 0, 0);
        }
        continue;
      }
      if constexpr (T::kScaled) {
        if (kk % 2 == 0) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
            sa[i] = *reinterpret_cast<const uint32_t*>(sc + (wm * C::WM + i * 32 + lrow) * C::SBPR + 4 * (kk / 2));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            sb[j] = *reinterpret_cast<const uint32_t*>(sc + (BM + wn * C::WN + j * 32 + lrow) * C::SBPR +
                                                       4 * (kk / 2));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) esa[i] = __builtin_amdgcn_ubfe(sa[i], 8 * (sbyte & 3), 8);
#pragma unroll
        for (int j = 0; j < TN; ++j) esb[j] = __builtin_amdgcn_ubfe(sb[j], 8 * (sbyte & 3), 8);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (FMT == 3) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fb[j][0]),
                                                                 __builtin_bit_cast(v8bf, fa[i][0]), acc[i][j], 0,
                                                                 0, 0);
          } else {
            const v4i qa0 = fa[i][0], qa1 = fa[i][NQ - 1];
            const v4i qb0 = fb[j][0], qb1 = fb[j][NQ - 1];
            const v8i a_op = FMT == 1 ? v8i{qa0.x, qa0.y, qa0.z, qa0.w, 0, 0, 0, 0}
                                      : v8i{qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
            const v8i b_op = FMT == 1 ? v8i{qb0.x, qb0.y, qb0.z, qb0.w, 0, 0, 0, 0}
                                      : v8i{qb0.x, qb0.y, qb0.z, qb0.w, qb1.x, qb1.y, qb1.z, qb1.w};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b_op, a_op, acc[i][j], T::kCbsz,
                                                                         T::kCbsz, 0, (int)esb[j], 0,
                                                                         (int)esa[i]);
          }
        }
    }
  };

  // Step s (unrolled position J = s % NSTG): load stage s + NSTG - 1 into
  // the buffer freed by step s - 1, compute stage s, then wait for this
  // wave's loads of stage s + 1 and for every wave.
  constexpr int kAhead = (NSTG - 2) * C::DW;
  auto step = [&](auto Jc, int s) {
    constexpr int J = decltype(Jc)::value;
    issue(smem + ((J + NSTG - 1) % NSTG) * C::STAGE, s + NSTG - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(smem + J * C::STAGE, T::kKK);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAhead) : "memory");
  };

#pragma unroll
  for (int t = 0; t < NSTG - 1; ++t) issue(smem + t * C::STAGE, t);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAhead) : "memory");

  int s = 0;
  for (; s + NSTG <= nfull; s += NSTG) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    if constexpr (NSTG > 2) step(std::integral_constant<int, 2>{}, s + 2);
    if constexpr (NSTG > 3) step(std::integral_constant<int, 3>{}, s + 3);
  }
  if (s < nfull) step(std::integral_constant<int, 0>{}, s++);
  if constexpr (NSTG > 2) {
    if (s < nfull) step(std::integral_constant<int, 1>{}, s++);
  }
  if constexpr (NSTG > 3) {
    if (s < nfull) step(std::integral_constant<int, 2>{}, s++);
  }
  // a partial last stage: already loaded (the previous wait covered it)
  if (tail_kk > 0) compute(smem + (nfull % NSTG) * C::STAGE, tail_kk);
  // past-end loads may still be landing in LDS that the epilogue reuses
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (KS == 2) {
    // the second K group's sums go through LDS to the first group's wave of
    // the same quadrant, which adds them to its own (first group + second,
    // a fixed order); the first group then runs the epilogue alone
    static_assert(WMW * WNW * TM * TN * 16 * 256 <= NSTG * C::STAGE, "exchange fits the stage buffers");
    float4* xch = reinterpret_cast<float4*>(smem) + (size_t)wg * TM * TN * 4 * 64;
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            xch[((i * TN + j) * 4 + g) * 64 + lane] =
                float4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 o = xch[((i * TN + j) * 4 + g) * 64 + lane];
            acc[i][j][4 * g] += o.x;
            acc[i][j][4 * g + 1] += o.y;
            acc[i][j][4 * g + 2] += o.z;
            acc[i][j][4 * g + 3] += o.w;
          }
    }
    __syncthreads();  // every read of the exchange is done before the strips reuse the LDS
    if (kg == 1) return;
  }

  // Epilogue.  The W tile is the MFMA's first operand, so the accumulator
  // is the transposed tile: lane l, element r holds row m = l % 32 of the A
  // tile and column n = 8 (r / 4) + 4 half + r % 4 of the W tile, i.e. four
  // consecutive columns of one output row per group r / 4.  Results go
  // through a per-wave LDS strip of 32 rows (BF16: the quadrant's full
  // width; FP32: half of it per pass where the quadrant is two or more MFMA
  // tiles wide), so every global store is a 16-byte chunk of a row.
  constexpr int WN = C::WN;                         // columns of a wave's quadrant
  constexpr int EB = EPI == kEpiStoreF32 ? 4 : 2;   // output element bytes
  // FP32 strips take two half-width passes when the quadrant has an even
  // number of 32-column MFMA tiles, else one full-width pass
  constexpr int NP = (EB == 4 && TN % 2 == 0) ? 2 : 1;  // passes per strip
  constexpr int SC = WN / NP;                           // strip columns per pass
  static_assert(TN % NP == 0 && SC % 32 == 0, "whole MFMA tiles per pass");
  constexpr int EPC = 16 / EB;                      // elements per 16-byte chunk
  constexpr int RSTR = SC * EB + 16;                // strip row stride in bytes (16-byte aligned)
  constexpr int CPR = SC * EB / 16;                 // chunks per strip row
  constexpr int RPI = 64 / CPR;                     // strip rows per wave-wide read (the last
                                                    // 64 - RPI * CPR lanes idle)
  constexpr int NRD = (32 + RPI - 1) / RPI;         // reads per strip
  static_assert(CPR % 4 == 0, "a lane quad holds one 32-column block of a row");
  static_assert(C::NW * 32 * RSTR <= NSTG * C::STAGE, "epilogue strips fit in the stage buffers");
  uint8_t* const strip = smem + wave * 32 * RSTR;
  const int n_wave = n0 + wn * WN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m_strip = m0 + wm * C::WM + i * 32;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int jj = 0; jj < TN / NP; ++jj) {
        const int j = p * (TN / NP) + jj;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint8_t* dst = strip + lrow * RSTR + (jj * 32 + 8 * g + 4 * half) * EB;
          if constexpr (EPI == kEpiStoreF32) {
            *reinterpret_cast<float4*>(dst) =
                float4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          } else {
            uint32_t b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              b[t] = pack_bf16(acc[i][j][4 * g + 2 * t], acc[i][j][4 * g + 2 * t + 1]);
              if constexpr (EPI == kEpiSiluBf16 || EPI == kEpiSiluQuant) {
                const float z0 = bf16_to_f32(b[t] & 0xFFFFu), z1 = bf16_to_f32(b[t] >> 16);
                b[t] = pack_bf16(silu_f32(z0), silu_f32(z1));
              }
            }
            *reinterpret_cast<uint2*>(dst) = uint2{b[0], b[1]};
          }
        }
      }
      // a wave's LDS accesses complete in order: the reads below see the
      // writes above, and the next pass's writes follow these reads
#pragma unroll
      for (int t = 0; t < NRD; ++t) {
        const int rho = t * RPI + lane / CPR, q = lane % CPR;
        if (lane >= RPI * CPR || rho >= 32) continue;  // whole rows, so whole quads
        const uint4 v = *reinterpret_cast<const uint4*>(strip + rho * RSTR + 16 * q);
        const int m = m_strip + rho, n = n_wave + p * SC + EPC * q;
        if (m >= M || n >= N) continue;
        if constexpr (EPI == kEpiSiluQuant) {
          // MX-quantize the BF16 u: lanes q = 4i .. 4i + 3 of a strip row
          // hold one 32-block (N % 32 == 0, so a quad is masked together),
          // encoded exactly as quant_rows_kernel does
          using Fq = typename std::conditional<FMT == 1, FmtE2M1, FmtE4M3>::type;
          const uint32_t sb = (uint32_t)(mx_block_exp<Fq>(quad_max(amax8(v))) + 127);
          uint8_t* crow = static_cast<uint8_t*>(Y) + (int64_t)m * (FMT == 1 ? N / 2 : N);
          encode_store8<Fq>(v, sb, crow + (FMT == 1 ? n / 2 : n));
          if ((q & 3) == 0) Ys[(int64_t)m * (N / 32) + n / 32] = (uint8_t)sb;
          continue;
        }
        const bool whole = N % EPC == 0 && n + EPC <= N;
        if constexpr (EPI == kEpiStoreF32) {
          float* yrow = reinterpret_cast<float*>(Y) + (int64_t)m * N;
          if (whole) {
            __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(yrow + n));
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 4; ++e)
              if (n + e < N) yrow[n + e] = __builtin_bit_cast(float, w[e]);
          }
        } else {
          uint16_t* yrow = reinterpret_cast<uint16_t*>(Y) + (int64_t)m * N;
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
          if constexpr (EPI == kEpiResAddBf16) {
            uint32_t h[4];
            if (whole) {
              const uint4 hv = *reinterpret_cast<const uint4*>(yrow + n);
              h[0] = hv.x, h[1] = hv.y, h[2] = hv.z, h[3] = hv.w;
            } else {
              for (int e = 0; e < 4; ++e) {
                const uint32_t lo = n + 2 * e < N ? yrow[n + 2 * e] : 0u;
                const uint32_t hi = n + 2 * e + 1 < N ? yrow[n + 2 * e + 1] : 0u;
                h[e] = lo | (hi << 16);
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[e] = pack_bf16(bf16_to_f32(h[e] & 0xFFFFu) + bf16_to_f32(w[e] & 0xFFFFu),
                               bf16_to_f32(h[e] >> 16) + bf16_to_f32(w[e] >> 16));
            }
          }
          if (whole) {
            // streaming store: the output is not read again by this kernel
            __builtin_nontemporal_store(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]},
                                        reinterpret_cast<v4i*>(yrow + n));
          } else {
            for (int e = 0; e < 8; ++e)
              if (n + e < N) yrow[n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

// The pipelined path applies when K is a whole number of MFMA slices whose
// stage scales are whole dwords in every row (K % 128 for MXFP4 and MXFP8,
// any K % 32 for BF16) and one tile's operand rows fit a 32-bit buffer
// range.
static int pipe_row_bytes(int fmt, int64_t K) {
  const int64_t q = fmt == 3 ? 32 : 128;
  return K % q == 0 ? 128 : 0;
}

bool gemm_pipe_supported(int fmt, int64_t M, int64_t N, int64_t K) {
  if (K <= 0 || pipe_row_bytes(fmt, K) == 0) return false;
  const int64_t ld = fmt == 1 ? K / 2 : (fmt == 3 ? 2 * K : K);
  return 256 * ld < (int64_t)0x7FFFFFFF && M > 0 && N > 0;
}

template <int FMT, int EPI, int BM, int BN, int RB, int WMW, int WNW, int NSTG, int KS = 1>
static hipError_t launch_pipe_t(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, uint8_t* ys, hipStream_t stream) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  gemm_pipe_kernel<FMT, EPI, BM, BN, RB, WMW, WNW, NSTG, KS><<<tm * tn, 64 * WMW * WNW * KS, 0, stream>>>(
      static_cast<const uint8_t*>(a), as, static_cast<const uint8_t*>(w), ws, (int)M, (int)N, (int)K, y, ys, tm,
      tn);
  return hipGetLastError();
}

template <int FMT, int EPI, int RB>
static hipError_t launch_pipe_r(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, uint8_t* ys, hipStream_t stream) {
  // 256 x 256 tiles (eight waves, two stages) when they fill the 256 CUs at
  // least once.  Small problems: 64 x 64 tiles (below).  Otherwise 128 x 128
  // tiles: three stages when one workgroup
  // per CU covers every tile (MXFP8 on four waves of 64 x 64, MXFP4 and BF16
  // on eight of 64 x 32: the faster layout of each, measured), else 256 x 128
  // tiles for long K (below), else two stages so that two workgroups share a
  // CU.
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 256) {
    // 256 x 192 tiles (4 x 2 waves of 64 x 96) when their rounds over the
    // 256 CUs cost less: a round of them is about 3/4 of a 256 x 256 round
    // (gate/up's N = 6144: 2 full rounds instead of 1.5)
    const int64_t mid = ((M + 255) / 256) * ((N + 191) / 192);
    if (3 * ((mid + 255) / 256) < 4 * ((big + 255) / 256))
      return launch_pipe_t<FMT, EPI, 256, 192, RB, 4, 2, 2>(a, as, w, ws, M, N, K, y, ys, stream);
    return launch_pipe_t<FMT, EPI, 256, 256, RB, 2, 4, 2>(a, as, w, ws, M, N, K, y, ys, stream);
  }
  const int64_t small = ((M + 127) / 128) * ((N + 127) / 128);
  // 128 x 128 tiles for at most half the CUs: 64 x 64 tiles (2 x 2 waves of
  // 32 x 32, three stages) spread the same work over four times the CUs
  // (128 x 1024 x 1024 MXFP4 5.5 -> 3.9 us, 512 x 1024 x 4096 MXFP8
  // 18.9 -> 9.3 us, 2048 x 1024 x 1024 BF16 10.1 -> 8.4 us).  With one
  // 128 x 128 tile per CU they move twice the operand bytes per FLOP and
  // lose (4096 x 1024 x 2048 MXFP8 14.0 -> 18.7 us).
  if (small <= 128) return launch_pipe_t<FMT, EPI, 64, 64, RB, 2, 2, 3>(a, as, w, ws, M, N, K, y, ys, stream);
  if constexpr (FMT == 2) {
    // exact MXFP8 with K of at least 24 stages: two K groups of 2 x 2 waves
    // of 64 x 64, each group taking every other slice, their sums added
    // through LDS before the epilogue.  Each wave's operand conversions then
    // feed two MFMAs where a 64 x 32 wave's feed one (4 instead of 6
    // conversions per MFMA, still two waves per SIMD).  4096 x 1024 x 3072:
    // 30.1 -> 28.2 us; at 16 stages (K = 2048) the exchange costs what the
    // conversions save.
    if (small <= 256 && K / 128 >= 24)
      return launch_pipe_t<FMT, EPI, 128, 128, RB, 2, 2, 3, 2>(a, as, w, ws, M, N, K, y, ys, stream);
  }
  if constexpr (FMT != 4) {
    if (small <= 256) return launch_pipe_t<FMT, EPI, 128, 128, RB, 2, 4, 3>(a, as, w, ws, M, N, K, y, ys, stream);
  }
  if (small <= 256) return launch_pipe_t<FMT, EPI, 128, 128, RB, 2, 2, 3>(a, as, w, ws, M, N, K, y, ys, stream);
  // More 128 x 128 tiles than CUs: 256 x 128 tiles (4 x 2 waves of 64 x 64,
  // three stages, one workgroup per CU) when they make a single round and K
  // spans at least 16 stages (the recurrent block's second GEMM, N = 2048,
  // K = 5632: 12-20% faster than two 128 x 128 workgroups per CU; at 8
  // stages or fewer they are no faster)
  const int64_t tall = ((M + 255) / 256) * ((N + 127) / 128);
  const int64_t stages = FMT == 1 ? K / 256 : FMT == 3 ? K / 64 : K / 128;
  if (tall <= 256 && stages >= 16)
    return launch_pipe_t<FMT, EPI, 256, 128, RB, 4, 2, 3>(a, as, w, ws, M, N, K, y, ys, stream);
  return launch_pipe_t<FMT, EPI, 128, 128, RB, 2, 2, 2>(a, as, w, ws, M, N, K, y, ys, stream);
}

template <int FMT, int EPI>
static hipError_t launch_pipe_e(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, uint8_t* ys, hipStream_t stream) {
  return launch_pipe_r<FMT, EPI, 128>(a, as, w, ws, M, N, K, y, ys, stream);
}

template <int FMT>
static hipError_t launch_pipe_f(int epi, const void* a, const uint8_t* as, const void* w, const uint8_t* ws,
                                int64_t M, int64_t N, int64_t K, void* y, uint8_t* ys, hipStream_t stream) {
  switch (epi) {
    case kEpiStoreBf16: return launch_pipe_e<FMT, kEpiStoreBf16>(a, as, w, ws, M, N, K, y, ys, stream);
    case kEpiStoreF32: return launch_pipe_e<FMT, kEpiStoreF32>(a, as, w, ws, M, N, K, y, ys, stream);
    case kEpiSiluBf16: return launch_pipe_e<FMT, kEpiSiluBf16>(a, as, w, ws, M, N, K, y, ys, stream);
    default: return launch_pipe_e<FMT, kEpiResAddBf16>(a, as, w, ws, M, N, K, y, ys, stream);
  }
}

hipError_t launch_gemm_pipe(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                            const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, hipStream_t stream) {
  if (fmt == 1) return launch_pipe_f<1>(epi, a, a_scales, w, w_scales, M, N, K, y, nullptr, stream);
  if (fmt == 2) return launch_pipe_f<2>(epi, a, a_scales, w, w_scales, M, N, K, y, nullptr, stream);
  if (fmt == 4) return launch_pipe_f<4>(epi, a, a_scales, w, w_scales, M, N, K, y, nullptr, stream);
  return launch_pipe_f<3>(epi, a, a_scales, w, w_scales, M, N, K, y, nullptr, stream);
}

hipError_t launch_gemm_silu_quant(int fmt, const void* a, const uint8_t* a_scales, const void* w,
                                  const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, uint8_t* codes,
                                  uint8_t* scales, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (N % 32 != 0 || !gemm_pipe_supported(fmt, M, N, K)) return hipErrorInvalidValue;
  if (fmt == 1) return launch_pipe_e<1, kEpiSiluQuant>(a, a_scales, w, w_scales, M, N, K, codes, scales, stream);
  if (fmt == 2) return launch_pipe_e<2, kEpiSiluQuant>(a, a_scales, w, w_scales, M, N, K, codes, scales, stream);
  if (fmt == 4) return launch_pipe_e<4, kEpiSiluQuant>(a, a_scales, w, w_scales, M, N, K, codes, scales, stream);
  return hipErrorInvalidValue;
}

}  // namespace rq
