// Pipelined block-scaled GEMM for gfx950: Y[M x N] = A . W^T, K-major.
//
// Same contraction as gemm.hip (ARCQuant unified GEMM; Day-0 page section V
// item 3: block scales applied inside the matrix core), organized for
// throughput on large problems:
//
// * A pipeline stage holds one RB-byte chunk (RB = 128, or 64 where K does
//   not divide) of every row of the A and W tiles: 2 RB elements of MXFP4,
//   RB of MXFP8 or RB / 2 of BF16, so each stage carries the same
//   matrix-core work whatever the format.  128-byte chunks are whole cache
//   lines for the global loads.
// * Global loads are buffer loads (the resource spans the tile's rows, so
//   rows past M or N read as zeros) into a ring of P register slots, issued
//   P stages ahead; each stage is then written to one of two LDS buffers
//   while the other feeds the MFMAs.  The loop is unrolled over the ring and
//   the two buffers so every register slot is static, and the compiler's
//   load counters wait exactly for the slot being written out.
// * LDS rows are RB bytes of 16-byte chunks, XOR-swizzled per row so that
//   the fragment reads of consecutive rows hit distinct banks (checked for
//   both 32- and 64-bank LDS models).
// * WMW x WNW waves, each owning a (BM/WMW) x (BN/WNW) quadrant of MFMA
//   tiles of 32 x 32; accumulators live in AGPRs.  256 x 256 tiles use
//   eight waves (two per SIMD, so one wave's waits and LDS writes overlap
//   the other's MFMAs), 128 x 128 tiles four (two workgroups share a CU).
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
#include <type_traits>

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
struct PipeTraits<3, RB> {  // BF16: RB / 2 K per stage in 16-deep slices
  static constexpr int kStepElems = RB / 2, kKK = RB / 32, kCbsz = 0, kSBPR = 0;
  static constexpr bool kScaled = false;
};

// Chunk swizzle of LDS row r.  64-byte rows: chunk bits (r1 ^ r3, r2 ^ r4);
// 128-byte rows: chunk bits (r0 ^ r3, r2, r1).
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB == 64)
    return ((r >> 1) ^ (r >> 3)) & 3;
  else
    return ((r ^ (r >> 3)) & 1) | ((r >> 1) & 2) | ((r << 1) & 4);
}

// Publish LDS writes and wait for every wave (no wait on global loads).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int FMT, int BM, int BN, int RB, int WMW, int WNW>
struct PipeCfg {
  using T = PipeTraits<FMT, RB>;
  static constexpr int NW = WMW * WNW, NT = 64 * NW;              // waves, threads
  static constexpr int TM = BM / 32 / WMW, TN = BN / 32 / WNW;    // MFMA tiles per wave
  static constexpr int WM = BM / WMW, WN = BN / WNW;              // wave quadrant
  static constexpr int CPR = RB / 16;                             // 16-byte chunks per row
  static constexpr int RPL = NT / CPR;                            // rows per workgroup-wide load
  static constexpr int CA = BM / RPL, CW = BN / RPL;              // 16-byte chunks per thread per stage
  static constexpr int SA = BM * RB, SW = BN * RB;                // LDS bytes of the A / W tile
  static constexpr int SBPR = T::kSBPR;                           // scale bytes per row per stage
  static constexpr int SS = (BM + BN) * SBPR;                     // scale bytes per stage
  static constexpr int STAGE = SA + SW + SS;
  static constexpr int NS = T::kScaled ? (BM + BN) / NT : 0;      // scale rows per thread
  static constexpr int SLOT = 4 * (CA + CW);                      // VGPRs of one ring slot
  // register ring depth: with two waves per SIMD three 16-VGPR slots or
  // one larger slot; otherwise one slot when it is large (the compiler
  // still renames it one stage ahead), two or four when small
  static constexpr int P = NW > 4 ? (SLOT <= 16 ? 3 : 1) : (SLOT >= 64 ? 1 : (SLOT >= 32 ? 2 : 4));
  static constexpr int U = P % 2 ? 2 * P : P;                     // steps per unrolled loop turn
  static_assert(CA * RPL == BM && CW * RPL == BN, "whole chunk rows per thread");
  static_assert(!T::kScaled || NS * NT == BM + BN, "whole scale rows per thread");
  static_assert(BM % 64 == 0, "A / W scale rows split on a wave boundary");
};

template <int SBPR>
struct ScaleWord {
  using type = uint32_t;
};
template <>
struct ScaleWord<8> {
  using type = uint2;
};

template <int FMT, int BM, int BN, int RB, int WMW, int WNW>
struct StageRegs {
  using C = PipeCfg<FMT, BM, BN, RB, WMW, WNW>;
  v4i a[C::CA];
  v4i w[C::CW];
  typename ScaleWord<C::SBPR>::type s[C::NS > 0 ? C::NS : 1];
};

template <int FMT, int EPI, int BM, int BN, int RB, int WMW, int WNW>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void gemm_pipe_kernel(const uint8_t* __restrict__ A,
                                                                      const uint8_t* __restrict__ As,
                                                                      const uint8_t* __restrict__ W,
                                                                      const uint8_t* __restrict__ Ws, int M, int N,
                                                                      int K, void* __restrict__ Y, int tiles_m,
                                                                      int tiles_n) {
  using C = PipeCfg<FMT, BM, BN, RB, WMW, WNW>;
  using T = PipeTraits<FMT, RB>;
  using SW_t = typename ScaleWord<C::SBPR>::type;
  constexpr int TM = C::TM, TN = C::TN, P = C::P, U = C::U;
  constexpr int CMAX = C::CA > C::CW ? C::CA : C::CW;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int half = lane >> 5, lrow = lane & 31;

  // XCD-aware tile order
  const int pid = blockIdx.x, nt = tiles_m * tiles_n;
  const int v = (nt % 8 == 0) ? (pid % 8) * (nt / 8) + pid / 8 : pid;
  constexpr int GM = 4;
  const int group = v / (GM * tiles_n), first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (v % (GM * tiles_n)) % gsz, tn = (v % (GM * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t ld = FMT == 1 ? (uint32_t)K / 2 : (FMT == 2 ? (uint32_t)K : 2u * (uint32_t)K);  // row bytes
  const uint32_t ksb = (uint32_t)K / 32;
  const int nk = K / T::kStepElems;

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

  // This thread's chunks: rows tid / CPR + RPL i, logical chunk tid % CPR.
  const int crow = tid / C::CPR, cchk = tid % C::CPR;
  uint32_t g_off[CMAX], l_off[CMAX];
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    const int r = crow + C::RPL * i;
    g_off[i] = (uint32_t)r * ld + 16u * (uint32_t)cchk;
    l_off[i] = (uint32_t)r * RB + 16u * (uint32_t)(cchk ^ swz<RB>(r));
  }

  StageRegs<FMT, BM, BN, RB, WMW, WNW> R[P];

  // Loads of stages past the end use an offset beyond every buffer range:
  // the hardware returns zeros without a memory access, so the prefetch
  // needs no branch (a branch around it would make the compiler's load
  // counter wait for everything at the join).
  constexpr uint32_t kPastEnd = 0x80000000u;
  auto load = [&](StageRegs<FMT, BM, BN, RB, WMW, WNW>& r, int s) {
    const uint32_t kb = s < nk ? (uint32_t)s * RB : kPastEnd;
#pragma unroll
    for (int i = 0; i < C::CA; ++i)
      r.a[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, g_off[i] + kb, 0, 0));
#pragma unroll
    for (int i = 0; i < C::CW; ++i)
      r.w[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, g_off[i] + kb, 0, 0));
    if constexpr (T::kScaled) {
      // Scale rows 0..BM-1 of A then 0..BN-1 of W, SBPR bytes per row and
      // load: thread t takes rows t + NT j; BM is a multiple of the wave
      // size, so the A / W choice is wave-uniform and the buffer resource
      // stays scalar.
      const uint32_t sk = s >= nk ? kPastEnd : (uint32_t)s * C::SBPR;
      auto ld_s = [&](__amdgpu_buffer_rsrc_t rs, uint32_t row) -> SW_t {
        if constexpr (C::SBPR == 8)
          return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, row * ksb + sk, 0, 0));
        else
          return __builtin_amdgcn_raw_buffer_load_b32(rs, row * ksb + sk, 0, 0);
      };
#pragma unroll
      for (int j = 0; j < C::NS; ++j) {
        const int rho = tid + C::NT * j;  // wave-uniform side
        if (__builtin_amdgcn_readfirstlane(rho) < BM)
          r.s[j] = ld_s(rsa, (uint32_t)rho);
        else
          r.s[j] = ld_s(rsw, (uint32_t)(rho - BM));
      }
    }
  };
  auto store = [&](const StageRegs<FMT, BM, BN, RB, WMW, WNW>& r, uint8_t* st) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) *reinterpret_cast<v4i*>(st + l_off[i]) = r.a[i];
#pragma unroll
    for (int i = 0; i < C::CW; ++i) *reinterpret_cast<v4i*>(st + C::SA + l_off[i]) = r.w[i];
    if constexpr (T::kScaled) {
#pragma unroll
      for (int j = 0; j < C::NS; ++j)
        *reinterpret_cast<SW_t*>(st + C::SA + C::SW + C::SBPR * (tid + C::NT * j)) = r.s[j];
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
  auto compute = [&](const uint8_t* st) {
    constexpr int KK = T::kKK;
    constexpr int NQ = FMT == 2 ? 2 : 1;  // 16-byte chunks per lane per fragment
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
      v4i fa[TM][NQ], fb[TN][NQ];
      // 16-byte chunk(s) of this slice for the lane's half
      const int c0 = FMT == 2 ? kk * 4 + half : kk * 2 + half;
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

  uint8_t* const lds0 = smem;
  uint8_t* const lds1 = smem + C::STAGE;

  // Step s (unrolled position J = s % U, register slot J % P): write stage
  // s+1 from its slot into the other LDS buffer, refill that slot with stage
  // s+1+P, compute stage s.
  auto step = [&](auto Jc, int s) {
    constexpr int J = decltype(Jc)::value;
    constexpr int Jn = (J + 1) % P;
    uint8_t* cur = (J % 2) ? lds1 : lds0;
    uint8_t* nxt = (J % 2) ? lds0 : lds1;
    store(R[Jn], nxt);  // past the last stage this writes zeros nobody reads
    // two waves per SIMD leave no registers to refill a one-slot ring
    // before it is written out
    if constexpr (C::NW > 4) __builtin_amdgcn_sched_barrier(0);
    load(R[Jn], s + 1 + P);
    // keep the refill ahead of the matrix work (the scheduler would sink it
    // below, shortening the prefetch distance by a step)
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
    lds_barrier();
  };

  // prologue: fill the ring, publish stage 0
#pragma unroll
  for (int t = 0; t < P; ++t) {
    load(R[t], t);
    // issue order = slot order, so the loop's per-slot load-count waits hold
    // on entry as well
    __builtin_amdgcn_sched_barrier(0);
  }
  store(R[0], lds0);
  load(R[0], P);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();

  int s = 0;
  for (; s + U <= nk; s += U) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    if constexpr (U > 2) step(std::integral_constant<int, 2>{}, s + 2);
    if constexpr (U > 3) step(std::integral_constant<int, 3>{}, s + 3);
    if constexpr (U > 4) step(std::integral_constant<int, 4>{}, s + 4);
    if constexpr (U > 5) step(std::integral_constant<int, 5>{}, s + 5);
  }
  // the last nk % U steps keep their unrolled positions (slot and buffer)
  if (s < nk) step(std::integral_constant<int, 0>{}, s++);
  if constexpr (U > 2) {
    if (s < nk) step(std::integral_constant<int, 1>{}, s++);
  }
  if constexpr (U > 3) {
    if (s < nk) step(std::integral_constant<int, 2>{}, s++);
  }
  if constexpr (U > 4) {
    if (s < nk) step(std::integral_constant<int, 3>{}, s++);
  }
  if constexpr (U > 5) {
    if (s < nk) step(std::integral_constant<int, 4>{}, s++);
  }

  // Epilogue.  The W tile is the MFMA's first operand, so the accumulator
  // is the transposed tile: lane l, element r holds row m = l % 32 of the A
  // tile and column n = 8 (r / 4) + 4 half + r % 4 of the W tile, i.e. four
  // consecutive columns of one output row per group r / 4.  Results go
  // through a per-wave LDS strip of 32 rows (BF16: the quadrant's full
  // width; FP32: half of it per pass), so every global store is a 16-byte
  // chunk of a row.
  constexpr int WN = C::WN;                         // columns of a wave's quadrant
  constexpr int EB = EPI == kEpiStoreF32 ? 4 : 2;   // output element bytes
  constexpr int SC = WN * 2 / EB;                   // strip columns per pass
  constexpr int NP = WN / SC;                       // passes per strip
  constexpr int EPC = 16 / EB;                      // elements per 16-byte chunk
  constexpr int RSTR = SC * EB + 16;                // strip row stride in bytes (16-byte aligned)
  constexpr int CPR = SC * EB / 16;                 // chunks per strip row
  constexpr int RPI = 64 / CPR;                     // strip rows per wave-wide read
  static_assert(C::NW * 32 * RSTR <= 2 * C::STAGE, "epilogue strips fit in the stage buffers");
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
            uint32_t b[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              uint32_t v = f32_to_bf16(acc[i][j][4 * g + t]);
              if constexpr (EPI == kEpiSiluBf16) {
                const float z = bf16_to_f32(v);
                v = f32_to_bf16(z / (1.0f + expf(-z)));
              }
              b[t] = v;
            }
            *reinterpret_cast<uint2*>(dst) = uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
          }
        }
      }
      // a wave's LDS accesses complete in order: the reads below see the
      // writes above, and the next pass's writes follow these reads
#pragma unroll
      for (int t = 0; t < 32 / RPI; ++t) {
        const int rho = t * RPI + lane / CPR, q = lane % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(strip + rho * RSTR + 16 * q);
        const int m = m_strip + rho, n = n_wave + p * SC + EPC * q;
        if (m >= M || n >= N) continue;
        const bool whole = N % EPC == 0 && n + EPC <= N;
        if constexpr (EPI == kEpiStoreF32) {
          float* yrow = reinterpret_cast<float*>(Y) + (int64_t)m * N;
          if (whole) {
            *reinterpret_cast<uint4*>(yrow + n) = v;
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
              const uint32_t lo = f32_to_bf16(bf16_to_f32(h[e] & 0xFFFFu) + bf16_to_f32(w[e] & 0xFFFFu));
              const uint32_t hi = f32_to_bf16(bf16_to_f32(h[e] >> 16) + bf16_to_f32(w[e] >> 16));
              w[e] = lo | (hi << 16);
            }
          }
          if (whole) {
            *reinterpret_cast<uint4*>(yrow + n) = uint4{w[0], w[1], w[2], w[3]};
          } else {
            for (int e = 0; e < 8; ++e)
              if (n + e < N) yrow[n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

// The pipelined path applies when K is a whole number of 64-byte stages
// (128-byte ones for MXFP8, whose scale rows must be whole dwords) and one
// tile's operand rows fit a 32-bit buffer range.  128-byte stages are used
// when K allows.
static int pipe_row_bytes(int fmt, int64_t K) {
  const int64_t e128 = fmt == 1 ? 256 : (fmt == 2 ? 128 : 64);
  const int64_t e64 = fmt == 1 ? 128 : (fmt == 2 ? 0 : 32);
  if (K % e128 == 0) return 128;
  if (e64 && K % e64 == 0) return 64;
  return 0;
}

bool gemm_pipe_supported(int fmt, int64_t M, int64_t N, int64_t K) {
  if (K <= 0 || pipe_row_bytes(fmt, K) == 0) return false;
  const int64_t ld = fmt == 1 ? K / 2 : (fmt == 2 ? K : 2 * K);
  return 256 * ld < (int64_t)0x7FFFFFFF && M > 0 && N > 0;
}

template <int FMT, int EPI, int BM, int BN, int RB, int WMW, int WNW>
static hipError_t launch_pipe_t(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, hipStream_t stream) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  gemm_pipe_kernel<FMT, EPI, BM, BN, RB, WMW, WNW><<<tm * tn, 64 * WMW * WNW, 0, stream>>>(
      static_cast<const uint8_t*>(a), as, static_cast<const uint8_t*>(w), ws, (int)M, (int)N, (int)K, y, tm, tn);
  return hipGetLastError();
}

template <int FMT, int EPI, int RB>
static hipError_t launch_pipe_r(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, hipStream_t stream) {
  // 256 x 256 tiles when they fill the 256 CUs at least once, else 128 x 128
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 256) return launch_pipe_t<FMT, EPI, 256, 256, RB, 2, 4>(a, as, w, ws, M, N, K, y, stream);
  return launch_pipe_t<FMT, EPI, 128, 128, RB, 2, 2>(a, as, w, ws, M, N, K, y, stream);
}

template <int FMT, int EPI>
static hipError_t launch_pipe_e(const void* a, const uint8_t* as, const void* w, const uint8_t* ws, int64_t M,
                                int64_t N, int64_t K, void* y, hipStream_t stream) {
  if constexpr (FMT == 2) {
    return launch_pipe_r<FMT, EPI, 128>(a, as, w, ws, M, N, K, y, stream);
  } else {
    if (pipe_row_bytes(FMT, K) == 128) return launch_pipe_r<FMT, EPI, 128>(a, as, w, ws, M, N, K, y, stream);
    return launch_pipe_r<FMT, EPI, 64>(a, as, w, ws, M, N, K, y, stream);
  }
}

template <int FMT>
static hipError_t launch_pipe_f(int epi, const void* a, const uint8_t* as, const void* w, const uint8_t* ws,
                                int64_t M, int64_t N, int64_t K, void* y, hipStream_t stream) {
  switch (epi) {
    case kEpiStoreBf16: return launch_pipe_e<FMT, kEpiStoreBf16>(a, as, w, ws, M, N, K, y, stream);
    case kEpiStoreF32: return launch_pipe_e<FMT, kEpiStoreF32>(a, as, w, ws, M, N, K, y, stream);
    case kEpiSiluBf16: return launch_pipe_e<FMT, kEpiSiluBf16>(a, as, w, ws, M, N, K, y, stream);
    default: return launch_pipe_e<FMT, kEpiResAddBf16>(a, as, w, ws, M, N, K, y, stream);
  }
}

hipError_t launch_gemm_pipe(int fmt, int epi, const void* a, const uint8_t* a_scales, const void* w,
                            const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, hipStream_t stream) {
  if (fmt == 1) return launch_pipe_f<1>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  if (fmt == 2) return launch_pipe_f<2>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
  return launch_pipe_f<3>(epi, a, a_scales, w, w_scales, M, N, K, y, stream);
}

}  // namespace rq
