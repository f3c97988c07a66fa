// gemm_mx.hip -- MXFP4 W4A4 prefill GEMM on gfx950's block-scaled FP4
// matrix cores ("MACaQ", core method: y = [(x*t)B]_MXFP4 W'^T_MXFP4).
//
// Each v_mfma_scale_f32_16x16x128_f8f6f4 (and its 32 x 32 x 64 form)
// consumes, per lane, 32 packed E2M1 codes of one row and the E8M0 byte of
// exactly that 32-element block, so the OCP MXFP4 tensors feed the
// instruction as stored: no dequantization.  The same template runs the
// exact-NVFP4 GEMM (fp16 matrix instructions after an exact dequantization)
// and the W4A16 GEMM (bf16).
//
// Data movement (the part that decides speed here):
//  * a 512-thread workgroup owns a BM x BN tile (MXFP4: 256 x 224 on
//    16 x 16 instructions, or 256 x 256 on 32 x 32); its eight wavefronts
//    (two per SIMD, so one wave's dequantization or LDS reads overlap the
//    other's matrix instructions) own 64 x BN/2 each;
//  * K advances 256 elements (one whole 128-byte line of codes per row) per
//    stage through a two-slot LDS ring filled by direct global->LDS loads
//    (global_load_lds, 16 bytes per lane) issued one stage ahead, so no
//    registers are spent on staging and the loads of stage k + 1 overlap
//    the matrix instructions of stage k (the NVFP4 and W4A16 forms issue
//    them in parts over the stage's first slices);
//  * a row's eight 16-byte chunks are stored XOR-swizzled by
//    (row ^ ((row >> 3) & 1)) & 7, which puts the 16-byte fragment reads of
//    16 consecutive rows on disjoint banks whether the LDS serves 128 or
//    256 bytes per clock;
//  * rows past M or N are loaded from the last valid row (their results are
//    never stored), so every lane issues the same number of loads and the
//    wait counts are compile-time constants;
//  * the fp32 output leaves through LDS: each wavefront re-stages 16-row
//    strips of its accumulators and writes whole rows with 16-byte stores
//    (scattered 4-byte lane stores ran at ~2.3 TB/s and cost as much time
//    as the whole K loop); the NVFP4 and W4A16 forms make those stores
//    non-temporal, the MXFP4 form ordinary (FP4Q_EPI_NT, FP4Q_EPI_NT_MX).

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>
#include <type_traits>

#include "internal.h"

#ifndef FP4Q_EPI_NT
#define FP4Q_EPI_NT 1           // non-temporal output stores: the GEMM is ~1% slower alone, but the fp32
                                // output no longer lingers dirty in the last-level cache, and the
                                // next step's quantizers run 10% faster (net ~1% per prefill step)
#endif
#ifndef FP4Q_EPI_NT_MX
#define FP4Q_EPI_NT_MX 0        // the MXFP4 GEMM keeps ordinary stores: 4.5% faster (78.4 against 82.1 us
                                // at 2048 x 14336 x 4096); the W4A16 GEMMs are 6% faster with
                                // non-temporal ones, like the NVFP4 step
#endif
#ifndef FP4Q_NV_SPREAD
#define FP4Q_NV_SPREAD 6        // NVFP4 next-stage loads in 6 parts over the first 6 of 8 slices: 5.9%
                                // faster at 4096 x 10240 x 5120 than all of them after the barrier
                                // (349.5 against 371.6 us; 4, 5, 7, 8 parts: 356-362 us); MXFP4
                                // gained nothing from spreading its loads
#endif
#ifndef FP4Q_W16_SPREAD
#define FP4Q_W16_SPREAD 6       // W4A16 (32 x 32 form, 8 slices) the same over 6 slices: the looped core's
                                // 13 GEMMs 4.5% faster grouped than with 3 parts (179.4 against 187.8 us;
                                // 2, 4, 7, 8 parts: 187.1, 183.0, 180.7, 184.1), 4% as single launches;
                                // the 16 x 16 form gained 7.4% from 3 parts over its 4 slices
#endif
#ifndef FP4Q_NV_SCHED_SPLIT
#define FP4Q_NV_SCHED_SPLIT 0   // 1: one scheduling region per 16-element block half
#endif

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

enum { FMT_MX = 0, FMT_NV = 1, FMT_W16 = 2 };   // W16: bf16 A, NVFP4 B
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// 8 NVFP4 codes -> 8 exact bf16 values code * s_b (at most 6 significant
// bits): the codes convert exactly to fp32, the fp32 product is exact and
// the upper halves are the bf16 values.  (gfx950 has no packed bf16
// multiply; the convert's own scale operand applies only the exponent.)
__device__ __forceinline__ v8bf dequant8_bf16(uint32_t w, float sb) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo, hi;
    switch (i) {
      case 0: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); lo = p[0]; hi = p[1]; break; }
      case 1: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); lo = p[0]; hi = p[1]; break; }
      case 2: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); lo = p[0]; hi = p[1]; break; }
      default: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); lo = p[0]; hi = p[1]; break; }
    }
    lo = lo * sb;
    hi = hi * sb;
    o[i] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, uint4{o[0], o[1], o[2], o[3]});
}

// Dword q (values 2q, 2q + 1) of dequant8_bf16, the same operations.
__device__ __forceinline__ uint32_t dequant2_bf16(uint32_t w, float sb, int q) {
  float lo, hi;
  switch (q) {
    case 0: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); lo = p[0]; hi = p[1]; break; }
    case 1: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); lo = p[0]; hi = p[1]; break; }
    case 2: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); lo = p[0]; hi = p[1]; break; }
    default: { auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); lo = p[0]; hi = p[1]; break; }
  }
  lo = lo * sb;
  hi = hi * sb;
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// E4M3 block scale (non-negative byte) -> the same value in fp16 (every
// E4M3 value, subnormals included, is an fp16 normal), splatted to both
// halves; one hardware fp8 -> fp16 convert.
__device__ __forceinline__ v2h e4m3_to_h2(uint32_t b) {
  const v2h t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false));
  return v2h{t[0], t[0]};
}

// 8 NVFP4 codes (one dword) -> 8 exact fp16 values code * s_b: the convert
// gives the code value exactly, the product has at most 2 + 4 significant
// bits and lies in [2^-10, 2688].
__device__ __forceinline__ v8h dequant8(uint32_t w, v2h sb) {
  const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * sb);
  const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * sb);
  const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * sb);
  const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * sb);
  return __builtin_bit_cast(v8h, uint4{o0, o1, o2, o3});
}

// Two of the eight values of dequant8 (dword q of its result), for
// splitting one fragment's dequantization across several instructions.
__device__ __forceinline__ uint32_t dequant2(uint32_t w, v2h sb, int q) {
  v2h t;
  switch (q) {
    case 0: t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)); break;
    case 1: t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)); break;
    case 2: t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)); break;
    default: t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)); break;
  }
  return __builtin_bit_cast(uint32_t, t * sb);
}

// vmcnt(n) for a wave-uniform n in [0, 31] (the count must be an immediate)
__device__ __forceinline__ void wait_vm(int n) {
#define FP4Q_VMW(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
  switch (n) {
    FP4Q_VMW(1) FP4Q_VMW(2) FP4Q_VMW(3) FP4Q_VMW(4) FP4Q_VMW(5) FP4Q_VMW(6) FP4Q_VMW(7) FP4Q_VMW(8)
    FP4Q_VMW(9) FP4Q_VMW(10) FP4Q_VMW(11) FP4Q_VMW(12) FP4Q_VMW(13) FP4Q_VMW(14) FP4Q_VMW(15) FP4Q_VMW(16)
    FP4Q_VMW(17) FP4Q_VMW(18) FP4Q_VMW(19) FP4Q_VMW(20) FP4Q_VMW(21) FP4Q_VMW(22) FP4Q_VMW(23) FP4Q_VMW(24)
    FP4Q_VMW(25) FP4Q_VMW(26) FP4Q_VMW(27) FP4Q_VMW(28) FP4Q_VMW(29) FP4Q_VMW(30) FP4Q_VMW(31)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
#undef FP4Q_VMW
}

struct MxArgs {
  const uint8_t* A;             // codes (MX, NV) or bf16 elements (W16)
  const uint8_t* As;
  const uint8_t* B;
  const uint8_t* Bs;
  const float* Ats;             // NVFP4 tensor scales (unused for MXFP4)
  const float* Bts;
  int64_t M, N, K;
  float* Y;
  int64_t ldy;
  int tiles_m, tiles_n;
  int64_t lda;                  // W16: row stride of A in elements
};

constexpr int GROUP_M = 8;

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  const int x = bid & 7, i = bid >> 3;
  const int base = nt >> 3, rem = nt & 7;
  const int t = x * base + (x < rem ? x : rem) + i;     // contiguous tile range per XCD
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int in_g = t - group * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// XOR swizzle of the 16-byte chunks of a staged row (CB / 16 chunks).  It
// depends on row % 16 only, so one value per lane serves every fragment,
// and it keeps the 16-byte reads of 16 consecutive rows on disjoint banks
// for 128- and 256-byte-per-clock LDS alike.
template <int CB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CB == 128) return (row ^ ((row >> 3) & 1)) & 7;
  else return ((row >> 1) ^ (row >> 3)) & 3;
}

// Direct global->LDS loads (gfx950 global_load_lds): lane l of the wave
// writes its 16 (or 4) bytes at LDS byte address m0 + 16 l (or 4 l).  They
// are issued from inline assembly so that the compiler does not serialise
// them against the LDS reads of other ring slots; ordering is explicit
// (s_waitcnt vmcnt + s_barrier below).  The instructions have no register
// results; the address registers are consumed at issue.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p);
}
// Address = uniform 64-bit base (SGPRs) + per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(off), "s"(base) : "memory");
}

// LDS stage layout and direct-load plan of one K stage for NT threads.  Each
// operand is a list of 16-byte (codes) or 4-byte (scales) units; unit s is
// loaded by thread s % NT in its load s / NT, and whole 64-unit groups
// belong to one wavefront, so "is this load present" is wave-uniform.
template <int FMT, int BM, int BN, int CB, int NT>
struct MxLayout {
  static constexpr int B_ROWS = BN;
  static constexpr int A_ROWB = FMT == FMT_W16 ? 4 * CB : CB;   // A bytes per row per stage
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + BM * A_ROWB;
  static constexpr int SA_OFF = B_OFF + B_ROWS * CB;
  static constexpr int SCB = FMT == FMT_MX ? CB / 16 : CB / 8;  // scale bytes per row per stage
  static constexpr int SA_ROWS = FMT == FMT_W16 ? 0 : BM;       // bf16 A has no scales
  static constexpr int SB_OFF = SA_OFF + SA_ROWS * SCB;
  static constexpr int STAGE = SB_OFF + B_ROWS * SCB;
  static constexpr int A_N = BM * A_ROWB / 16, B_N = B_ROWS * CB / 16;      // 16-byte units
  static constexpr int SA_N = SA_ROWS * SCB / 4, SB_N = B_ROWS * SCB / 4;    // 4-byte units
  static constexpr int A_LD = (A_N + NT - 1) / NT, B_LD = (B_N + NT - 1) / NT;
  static constexpr int SA_LD = (SA_N + NT - 1) / NT, SB_LD = (SB_N + NT - 1) / NT;
  static_assert(A_N % 64 == 0 && B_N % 64 == 0 && SA_N % 64 == 0 && SB_N % 64 == 0, "whole-wave loads");
};

// NW wavefronts in a (NW / 2) x 2 grid over the tile; NS ring slots.
// M32 = 1: 32 x 32 matrix instructions (v_mfma_scale_f32_32x32x64_f8f6f4,
// v_mfma_f32_32x32x16_f16), which sustain about twice the rate of the
// 16 x 16 shapes on gfx950 (measured: 9.4 vs 5.0 PFLOP/s for FP4, 2.4 vs
// 1.4 for fp16 with independent accumulators); lane l then serves row
// l % 32 and K half l / 32, and accumulator register r holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// One output tile (index bid of p's tiles) per call; the kernels below
// map workgroups to (problem, tile).
template <int FMT, int BM, int BN, int CB, int NW, int NS, int M32>
__device__ __forceinline__ void mx3_tile(const MxArgs& p, int bid) {
  constexpr int NT = NW * 64;
  using Lay = MxLayout<FMT, BM, BN, CB, NT>;
  constexpr int CPR = CB / 16;                    // 16-byte chunks per staged row
  constexpr int KS = CB / 64;                     // 128-element instruction steps per stage
  constexpr int WM = NW / 2, RW = BM / WM;        // wavefront rows, rows per wavefront
  static_assert(BM % 64 == 0 && BM <= 512 && BN % 32 == 0 && BN <= 320 && (CB == 64 || CB == 128), "tile");
  static_assert((NW == 4 || NW == 8) && NS >= 2 && NS <= 4 && RW % 16 == 0, "layout");
  static_assert(!M32 || (RW % 32 == 0 && (BN / 2) % 32 == 0), "32 x 32 tiles");
  constexpr int TS = M32 ? 32 : 16;               // accumulator tile edge
  constexpr int FM = RW / TS, FN = BN / (2 * TS);
  using Acc = typename std::conditional<M32 != 0, v16f, v4f>::type;
  // the ring, and after the K loop the epilogue's 16-row staging strips
  constexpr int EPI = NW * 16 * (BN / 2 + 4) * 4;
  constexpr int SMEM = NS * Lay::STAGE > EPI ? NS * Lay::STAGE : EPI;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 4, r16 = lane & 15;
  const int r32 = lane & 31, hh = lane >> 5;      // 32 x 32 instructions: row, K half
  int tm, tn;
  tile_of(bid, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t ldb = p.K / 2, lds = p.K / (FMT == FMT_MX ? 32 : 16);
  const int KT = (int)(p.K / (2 * CB));

  // ---- per-thread byte offsets of the direct loads (row and chunk are
  // fixed over K; the stage adds kt * 128 bytes of codes / 8 of scales).
  uint32_t offA[Lay::A_LD], offB[Lay::B_LD], offSA[Lay::SA_LD > 0 ? Lay::SA_LD : 1], offSB[Lay::SB_LD];
#pragma unroll
  for (int i = 0; i < Lay::A_LD; ++i) {
    if constexpr (FMT == FMT_W16) {
      // bf16 rows of 4 CB bytes per stage; 16-byte chunk c of row r is
      // stored at position c ^ (r % 16), so the 16 rows a fragment read
      // touches fall on 16 different positions
      constexpr int CPA = Lay::A_ROWB / 16;
      const int s = i * NT + tid, row = s / CPA, gch = (s % CPA) ^ (row & 15);
      int64_t r = m0 + row;
      r = r < p.M ? r : p.M - 1;
      offA[i] = (uint32_t)(r * p.lda * 2 + gch * 16);
    } else {
      const int s = i * NT + tid, row = s / CPR, gch = (s % CPR) ^ swz<CB>(row);
      int64_t r = m0 + row;
      r = r < p.M ? r : p.M - 1;
      offA[i] = (uint32_t)(r * ldb + gch * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < Lay::B_LD; ++i) {
    const int s = i * NT + tid, row = s / CPR, gch = (s % CPR) ^ swz<CB>(row);
    int64_t r = n0 + row;
    r = r < p.N ? r : p.N - 1;
    offB[i] = (uint32_t)(r * ldb + gch * 16);
  }
  // scales: SCB bytes per row per stage, one 4-byte word per lane
  constexpr int WPR = Lay::SCB / 4;               // words per row per stage
#pragma unroll
  for (int i = 0; i < Lay::SA_LD; ++i) {
    const int s = i * NT + tid;
    int64_t r = m0 + s / WPR;
    r = r < p.M ? r : p.M - 1;
    offSA[i] = (uint32_t)(r * lds + (s % WPR) * 4);
  }
#pragma unroll
  for (int i = 0; i < Lay::SB_LD; ++i) {
    const int s = i * NT + tid;
    int64_t r = n0 + s / WPR;
    r = r < p.N ? r : p.N - 1;
    offSB[i] = (uint32_t)(r * lds + (s % WPR) * 4);
  }

  const uint32_t smem_base = lds_offset(smem);
  // Issues this wavefront's loads of stage kt whose index in the list
  // (A units, B units, A scale words, B scale words) is `part` modulo P;
  // P = 1 issues them all.
  auto issue = [&](int kt, int part = 0, int P = 1) {
    const uint32_t st = smem_base + (uint32_t)((kt % NS) * Lay::STAGE);
    const uint32_t kc = (uint32_t)kt * CB, ksc = (uint32_t)kt * Lay::SCB, kca = (uint32_t)kt * Lay::A_ROWB;
    int idx = 0;
#pragma unroll
    for (int i = 0; i < Lay::A_LD; ++i, ++idx)
      if (idx % P == part && i * NT + wave * 64 < Lay::A_N)       // wave-uniform
        dma16(p.A, offA[i] + kca, st + Lay::A_OFF + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < Lay::B_LD; ++i, ++idx)
      if (idx % P == part && i * NT + wave * 64 < Lay::B_N)
        dma16(p.B, offB[i] + kc, st + Lay::B_OFF + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < Lay::SA_LD; ++i, ++idx)
      if (idx % P == part && i * NT + wave * 64 < Lay::SA_N)
        dma4(p.As, offSA[i] + ksc, st + Lay::SA_OFF + (i * NT + wave * 64) * 4);
#pragma unroll
    for (int i = 0; i < Lay::SB_LD; ++i, ++idx)
      if (idx % P == part && i * NT + wave * 64 < Lay::SB_N)
        dma4(p.Bs, offSB[i] + ksc, st + Lay::SB_OFF + (i * NT + wave * 64) * 4);
  };
  // NVFP4 on 32 x 32 instructions and W4A16 issue the next stage's loads
  // in SPREAD parts, one at the start of each of the stage's first SPREAD
  // slices (NVFP4: CB / 32 steps of four 16-K instructions; W4A16: 8-element
  // slices of the two block halves), instead of all of them right after the
  // barrier: every wavefront then waits less for the address unit to take
  // its loads before it can go on with its own multiplies.
  constexpr int SPREAD = (FMT == FMT_NV && M32) ? FP4Q_NV_SPREAD : FMT == FMT_W16 ? FP4Q_W16_SPREAD : 0;
  static_assert(SPREAD <= (M32 ? CB / 32 * 4 : KS * 4), "one part per slice at most");
  // loads this wavefront issues per stage (wave-uniform)
  int nload = 0;
#pragma unroll
  for (int i = 0; i < Lay::A_LD; ++i) nload += (i * NT + wave * 64 < Lay::A_N);
#pragma unroll
  for (int i = 0; i < Lay::B_LD; ++i) nload += (i * NT + wave * 64 < Lay::B_N);
#pragma unroll
  for (int i = 0; i < Lay::SA_LD; ++i) nload += (i * NT + wave * 64 < Lay::SA_N);
#pragma unroll
  for (int i = 0; i < Lay::SB_LD; ++i) nload += (i * NT + wave * 64 < Lay::SB_N);

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

  // Stage kt lives in ring slot kt % NS, and NS - 1 stages are loaded
  // ahead.  At the top of iteration kt the wait leaves only the later
  // stages' loads in flight; after the barrier stage kt is visible to every
  // wave and every wave has finished reading stage kt - 1, whose slot then
  // receives stage kt + NS - 1.  (A plain s_barrier, not __syncthreads: its
  // release fence would also wait for loads that are meant to stay in
  // flight.)
#pragma unroll
  for (int k = 0; k < NS - 1; ++k)
    if (k < KT) issue(k);
  for (int kt = 0; kt < KT; ++kt) {
    const int ahead = min(KT - 1 - kt, NS - 2);
    wait_vm(ahead * nload);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const bool more = kt + NS - 1 < KT;                // a stage is left to load
    if constexpr (SPREAD == 0)
      if (more) issue(kt + NS - 1);
    if constexpr (FMT == FMT_MX && M32) {
      // Step ks covers K elements [64 ks, 64 ks + 64) of the stage; lane half
      // hh reads 16-byte chunk 2 ks + hh of its row: one 32-element MXFP4
      // block, whose scale byte has the same index.  A fragments first, then
      // the B fragments one column block ahead of their multiplies.
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < CB / 32; ++ks) {
        const int c = 2 * ks + hh;
        v8i fa[FM];
        int fsa[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * RW + i * 32 + r32;
          const uint4 q = *reinterpret_cast<const uint4*>(st + Lay::A_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
          fa[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          fsa[i] = st[Lay::SA_OFF + row * Lay::SCB + c];
        }
        auto ldb = [&](int j, v8i& fb, int& fsb) {
          const int row = wn * (BN / 2) + j * 32 + r32;
          const uint4 q = *reinterpret_cast<const uint4*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
          fb = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          fsb = st[Lay::SB_OFF + row * Lay::SCB + c];
        };
        v8i fb[2];
        int fsb[2];
        ldb(0, fb[0], fsb[0]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (j + 1 < FN) ldb(j + 1, fb[(j + 1) & 1], fsb[(j + 1) & 1]);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j & 1], acc[i][j], 4, 4, 0, fsa[i],
                                                                        0, fsb[j & 1]);
        }
        // the same scheduling groups as the 16 x 16 path below (without
        // them this path was 3-8% slower than that one; with them 3-5%
        // faster on the same tiles)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM + 2, 0);          // A blocks, B block 0
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (j + 1 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // B block j + 1
          __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                // block j's multiplies
        }
      }
    } else if constexpr (FMT == FMT_MX) {
      // Instruction step ks covers K elements [128 ks, 128 ks + 128) of the
      // stage; lane group g reads 16-byte chunk 4 ks + g of its row.  The A
      // fragments of the step are read first, then the B fragments one
      // column block at a time, so that the read of block j + 1 is in flight
      // while block j multiplies (measured 2% faster than reading all
      // fragments of the step before the first multiply).
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + g;
        v8i fa[FM];
        int fsa[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * RW + i * 16 + r16;
          const uint4 q = *reinterpret_cast<const uint4*>(st + Lay::A_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
          fa[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          fsa[i] = st[Lay::SA_OFF + row * Lay::SCB + c];
        }
        auto ldb = [&](int j, v8i& fb, int& fsb) {
          const int row = wn * (BN / 2) + j * 16 + r16;
          const uint4 q = *reinterpret_cast<const uint4*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
          fb = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          fsb = st[Lay::SB_OFF + row * Lay::SCB + c];
        };
        v8i fb[2];
        int fsb[2];
        ldb(0, fb[0], fsb[0]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (j + 1 < FN) ldb(j + 1, fb[(j + 1) & 1], fsb[(j + 1) & 1]);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j & 1], acc[i][j], 4, 4, 0, fsa[i],
                                                                         0, fsb[j & 1]);
        }
        // Scheduling groups that keep the reads of B block j + 1 (codes
        // and scale byte) ahead of block j's multiplies.  Left alone, the
        // scheduler issued each read after the multiplies of the block
        // before, into the same registers, and every block then waited
        // for its read (the groups: 1.9-3.6% faster, bit-identical).
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM + 2, 0);          // A blocks, B block 0
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (j + 1 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // B block j + 1
          __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                // block j's multiplies
        }
      }
    } else if constexpr (FMT == FMT_W16 && M32) {
      // bf16 A x NVFP4 B on 32 x 32 x 16 bf16 instructions, with the K
      // assignment of the NVFP4 32 x 32 path: step ks, lane half hh -> B
      // chunk c = 2 ks + hh, its dword t -> instruction t; the matching 8 bf16
      // values of A are its staged 16-byte chunk 8 ks + 4 hh + t
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < CB / 32; ++ks) {
        const int c = 2 * ks + hh;
        uint32_t rb[FN];                               // scale pairs first, as in the NVFP4 path
#pragma unroll
        for (int j = 0; j < FN; ++j)
          rb[j] = *reinterpret_cast<const uint16_t*>(st + Lay::SB_OFF + (wn * (BN / 2) + j * 32 + r32) * Lay::SCB + 2 * c);
        uint4 qb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * (BN / 2) + j * 32 + r32;
          qb[j] = *reinterpret_cast<const uint4*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
        }
        float sbf[FN][2];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const auto sp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(rb[j], 1.0f, false);
          sbf[j][0] = sp[0];
          sbf[j][1] = sp[1];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (ks | t) __builtin_amdgcn_sched_barrier(0);
          if constexpr (SPREAD > 0)
            if (ks * 4 + t < SPREAD && more) issue(kt + NS - 1, ks * 4 + t, SPREAD);
          v8bf ha[FM];
          const int ch = 8 * ks + 4 * hh + t;          // bf16 chunk within the staged row
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int row = wm * RW + i * 32 + r32;
            ha[i] = *reinterpret_cast<const v8bf*>(st + Lay::A_OFF + row * Lay::A_ROWB + ((ch ^ (row & 15)) << 4));
          }
          __builtin_amdgcn_s_setprio(1);
          // B block j + 1 dequantized in FM parts behind block j's multiplies,
          // into the other of two register sets
          uint32_t hb[2][4];
          {
            const uint32_t w = t == 0 ? qb[0].x : t == 1 ? qb[0].y : t == 2 ? qb[0].z : qb[0].w;
#pragma unroll
            for (int q = 0; q < 4; ++q) hb[0][q] = dequant2_bf16(w, sbf[0][t >> 1], q);
          }
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v8bf cur = __builtin_bit_cast(v8bf, uint4{hb[j & 1][0], hb[j & 1][1], hb[j & 1][2], hb[j & 1][3]});
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[i], cur, acc[i][j], 0, 0, 0);
              if (j + 1 < FN) {
                const int jn = j + 1 < FN ? j + 1 : j;
                const uint32_t w = t == 0 ? qb[jn].x : t == 1 ? qb[jn].y : t == 2 ? qb[jn].z : qb[jn].w;
#pragma unroll
                for (int q = i * 4 / FM; q < (i + 1) * 4 / FM; ++q) hb[(j + 1) & 1][q] = dequant2_bf16(w, sbf[jn][t >> 1], q);
              }
            }
          }
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one matrix instruction
              if (j + 1 < FN) __builtin_amdgcn_sched_group_barrier(0x002, 16 / FM, 0);  // then VALU
            }
          __builtin_amdgcn_s_setprio(0);
        }
      }
    } else if constexpr (FMT == FMT_W16) {
      // bf16 A x NVFP4 B: the same K assignment as the NVFP4 path (lane
      // group g, block half h, slice s2 -> elements 32 c + 16 h + 8 s2 of
      // chunk c), A read as 16-byte bf16 chunks, B dequantized exactly to
      // bf16, bf16 matrix core
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint2 qb[FN];
          float sbf[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int row = wn * (BN / 2) + j * 16 + r16;
            qb[j] = *reinterpret_cast<const uint2*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4) + 8 * h);
            sbf[j] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st[Lay::SB_OFF + row * Lay::SCB + 2 * c + h], 1.0f, false)[0];
          }
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if constexpr (SPREAD > 0)
              if ((ks * 2 + h) * 2 + s2 < SPREAD && more) issue(kt + NS - 1, (ks * 2 + h) * 2 + s2, SPREAD);
            v8bf ha[FM];
            const int ch = 16 * ks + 4 * g + 2 * h + s2;     // bf16 chunk within the staged row
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              const int row = wm * RW + i * 16 + r16;
              ha[i] = *reinterpret_cast<const v8bf*>(st + Lay::A_OFF + row * Lay::A_ROWB + ((ch ^ (row & 15)) << 4));
            }
            __builtin_amdgcn_s_setprio(1);      // as in the NVFP4 path
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const v8bf hb = dequant8_bf16(s2 ? qb[j].y : qb[j].x, sbf[j]);
#pragma unroll
              for (int i = 0; i < FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[i], hb, acc[i][j], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
          }
        }
      }
    } else if constexpr (M32) {
      // NVFP4, 32 x 32 x 16 fp16 instructions: step ks covers K elements
      // [64 ks, 64 ks + 64) of the stage; lane half hh reads 16-byte chunk
      // c = 2 ks + hh of its row (two 16-element blocks, scale bytes 2c and
      // 2c + 1) and feeds its dwords t = 0..3 (8 elements each) to
      // instruction t; A and B use the same assignment, so each instruction
      // sums over matching K elements.
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < CB / 32; ++ks) {
        const int c = 2 * ks + hh;
        // scale pairs first, then codes: the scale conversions then wait
        // only for the small reads, not for every code read behind them
        // (reads interleaved per block: 3.4% slower at 4096 x 10240 x 5120)
        uint32_t ra[FM], rb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          ra[i] = *reinterpret_cast<const uint16_t*>(st + Lay::SA_OFF + (wm * RW + i * 32 + r32) * Lay::SCB + 2 * c);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          rb[j] = *reinterpret_cast<const uint16_t*>(st + Lay::SB_OFF + (wn * (BN / 2) + j * 32 + r32) * Lay::SCB + 2 * c);
        uint4 qa[FM];
        v2h sa[FM][2];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * RW + i * 32 + r32;
          qa[i] = *reinterpret_cast<const uint4*>(st + Lay::A_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
        }
        uint4 qb[FN];
        v2h sb[FN][2];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * (BN / 2) + j * 32 + r32;
          qb[j] = *reinterpret_cast<const uint4*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const v2h t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ra[i], 1.0f, false));
          sa[i][0] = v2h{t[0], t[0]};
          sa[i][1] = v2h{t[1], t[1]};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v2h t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rb[j], 1.0f, false));
          sb[j][0] = v2h{t[0], t[0]};
          sb[j][1] = v2h{t[1], t[1]};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (ks | t) __builtin_amdgcn_sched_barrier(0);
          if constexpr (SPREAD > 0)
            if (ks * 4 + t < SPREAD && more) issue(kt + NS - 1, ks * 4 + t, SPREAD);
          v8h ha[FM];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint32_t w = t == 0 ? qa[i].x : t == 1 ? qa[i].y : t == 2 ? qa[i].z : qa[i].w;
            ha[i] = dequant8(w, sa[i][t >> 1]);
          }
          __builtin_amdgcn_s_setprio(1);
          // B fragment j + 1 is dequantized in FM parts, one after each
          // multiply of fragment j, into the other of two register sets; the
          // scheduling groups below keep that one-multiply, few-VALU rhythm
          // (measured 1% faster than dequantizing each fragment whole
          // before its multiplies; results bit-identical)
          uint32_t hb[2][4];
          {
            const uint32_t w = t == 0 ? qb[0].x : t == 1 ? qb[0].y : t == 2 ? qb[0].z : qb[0].w;
#pragma unroll
            for (int q = 0; q < 4; ++q) hb[0][q] = dequant2(w, sb[0][t >> 1], q);
          }
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v8h cur = __builtin_bit_cast(v8h, uint4{hb[j & 1][0], hb[j & 1][1], hb[j & 1][2], hb[j & 1][3]});
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[i], cur, acc[i][j], 0, 0, 0);
              if (j + 1 < FN) {
                const int jn = j + 1 < FN ? j + 1 : j;
                const uint32_t w = t == 0 ? qb[jn].x : t == 1 ? qb[jn].y : t == 2 ? qb[jn].z : qb[jn].w;
#pragma unroll
                for (int q = i * 4 / FM; q < (i + 1) * 4 / FM; ++q) hb[(j + 1) & 1][q] = dequant2(w, sb[jn][t >> 1], q);
              }
            }
          }
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one matrix instruction
              if (j + 1 < FN) __builtin_amdgcn_sched_group_barrier(0x002, 8 / FM, 0);   // then VALU
            }
          __builtin_amdgcn_s_setprio(0);
        }
      }
    } else {
      // NVFP4: lane group g owns elements [32 c, 32 c + 32) of chunk c; each
      // half h is one 16-element block, consumed as two 8-element slices by
      // the fp16 instruction (the same element assignment for A and B).
      const uint8_t* st = smem + (kt % NS) * Lay::STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#if FP4Q_NV_SCHED_SPLIT
          if (ks | h) __builtin_amdgcn_sched_barrier(0);
#endif
          uint2 qa[FM];
          v2h sa[FM];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int row = wm * RW + i * 16 + r16;
            qa[i] = *reinterpret_cast<const uint2*>(st + Lay::A_OFF + row * CB + ((c ^ swz<CB>(row)) << 4) + 8 * h);
            sa[i] = e4m3_to_h2(st[Lay::SA_OFF + row * Lay::SCB + 2 * c + h]);
          }
          uint2 qb[FN];
          v2h sb[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int row = wn * (BN / 2) + j * 16 + r16;
            qb[j] = *reinterpret_cast<const uint2*>(st + Lay::B_OFF + row * CB + ((c ^ swz<CB>(row)) << 4) + 8 * h);
            sb[j] = e4m3_to_h2(st[Lay::SB_OFF + row * Lay::SCB + 2 * c + h]);
          }
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            v8h ha[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) ha[i] = dequant8(s2 ? qa[i].y : qa[i].x, sa[i]);
            // raised wave priority for the matrix instructions: the wavefront
            // in its multiply block goes first, so the two wavefronts of a
            // SIMD drift apart and one's dequantization overlaps the other's
            // multiplies (measured +1%)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const v8h hb = dequant8(s2 ? qb[j].y : qb[j].x, sb[j]);
#pragma unroll
              for (int i = 0; i < FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[i], hb, acc[i][j], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
          }
        }
      }
    }
  }

  // ---- epilogue: each wavefront stages one 16-row strip of its tile at a
  // time in its own LDS area and writes whole rows with 16-byte stores
  // (the fp32 output is the largest stream of the kernel).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();                   // ring slots no longer read
  constexpr int WC = BN / 2;                      // columns per wavefront
  constexpr int LDE = WC + 4;                     // padded staging row (floats)
  float* stage = reinterpret_cast<float*>(smem) + wave * 16 * LDE;
  const int64_t col0 = n0 + wn * WC;
  const bool vec = ((p.ldy & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.Y) & 15) == 0);
  const float tsc = FMT == FMT_NV ? (*p.Ats) * (*p.Bts) : FMT == FMT_W16 ? *p.Bts : 1.0f;
  // writes the 16 x WC strip staged in `stage` to output rows row0 .. +15
  auto write_strip = [&](int64_t row0) {
#pragma unroll
    for (int k = 0; k < (16 * WC / 4 + 63) / 64; ++k) {
      const int idx = k * 64 + lane;
      if (idx < 16 * WC / 4) {
        const int rr = idx / (WC / 4), c4 = (idx % (WC / 4)) * 4;
        const v4f v = *reinterpret_cast<const v4f*>(&stage[rr * LDE + c4]);
        const int64_t row = row0 + rr, col = col0 + c4;
        if (row < p.M) {
          float* dst = p.Y + row * p.ldy + col;
          if (vec && col + 4 <= p.N) {
            if constexpr ((FMT == FMT_MX ? FP4Q_EPI_NT_MX : FP4Q_EPI_NT) != 0)
              __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(dst));
            else
              *reinterpret_cast<v4f*>(dst) = v;
          } else {
            if (col + 0 < p.N) dst[0] = v[0];
            if (col + 1 < p.N) dst[1] = v[1];
            if (col + 2 < p.N) dst[2] = v[2];
            if (col + 3 < p.N) dst[3] = v[3];
          }
        }
      }
    }
  };
  if constexpr (M32) {
    // 32-row tiles leave as two 16-row strips: register r of lane l holds
    // tile row 8 (r / 4) + 4 (l / 32) + r % 4, so strip q takes r in
    // [8 q, 8 q + 8)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r8 = 0; r8 < 8; ++r8) {
            float v = acc[i][j][8 * q + r8];
            if constexpr (FMT != FMT_MX) v = v * tsc;
            stage[(8 * (r8 >> 2) + 4 * hh + (r8 & 3)) * LDE + j * 32 + r32] = v;
          }
        write_strip(m0 + wm * RW + i * 32 + 16 * q);
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[i][j][r];
          if constexpr (FMT != FMT_MX) v = v * tsc;
          stage[(g * 4 + r) * LDE + j * 16 + r16] = v;
        }
      write_strip(m0 + wm * RW + i * 16);
    }
  }
}

template <int FMT, int BM, int BN, int CB, int MINB, int NW, int NS, int M32>
__global__ __launch_bounds__(NW * 64, MINB) void k_gemm_mx3(const MxArgs p) {
  mx3_tile<FMT, BM, BN, CB, NW, NS, M32>(p, (int)blockIdx.x);
}

// Several problems of one format in one launch: workgroups
// [start[i], start[i + 1]) take the tiles of problem i.
constexpr int kMaxGroup = 16;
struct MxGroup {
  MxArgs prob[kMaxGroup];
  int start[kMaxGroup + 1];
  int n;
};

template <int FMT, int BM, int BN, int CB, int MINB, int NW, int NS, int M32>
__global__ __launch_bounds__(NW * 64, MINB) void k_gemm_mx3_grouped(const MxGroup grp) {
  int i = 0;
  while (i + 1 < grp.n && (int)blockIdx.x >= grp.start[i + 1]) ++i;
  mx3_tile<FMT, BM, BN, CB, NW, NS, M32>(grp.prob[i], (int)blockIdx.x - grp.start[i]);
}

#ifndef FP4Q_MX_M32
#define FP4Q_MX_M32 1         // 256-wide tiles on 32 x 32 x 64 FP4 instructions: 4.8% faster than
                              // 16 x 16 x 128 at 2048 x 16384 x 4096 (92.8 against 97.5 us); the
                              // 224-wide tiles (2048 x 14336) stay on 16 x 16, which 224 / 2 needs
#endif
#ifndef FP4Q_MX_BN
#define FP4Q_MX_BN 256        // workgroup columns (16 x 16 path: 224 for widths that 224 divides and 256 does not)
#endif
#ifndef FP4Q_MX_BM
#define FP4Q_MX_BM 256        // workgroup rows
#endif
#ifndef FP4Q_MX_CB
#define FP4Q_MX_CB 128        // code bytes per row per stage
#endif
#ifndef FP4Q_MX_MINB
#define FP4Q_MX_MINB 1        // workgroups per CU the register budget targets
#endif
#ifndef FP4Q_MX_NW
#define FP4Q_MX_NW 8          // wavefronts per workgroup
#endif
#ifndef FP4Q_MX_NS
#define FP4Q_MX_NS 2          // LDS ring slots
#endif
#ifndef FP4Q_NV_M32
#define FP4Q_NV_M32 1         // 32 x 32 x 16 fp16 instructions on 256 x 128 tiles: 4-6% faster than
                              // 16 x 16 x 32 on 256 x 160 (0)
#endif
#ifndef FP4Q_NV_BM
#define FP4Q_NV_BM 256
#endif
#ifndef FP4Q_NV_BN
#if FP4Q_NV_M32
#define FP4Q_NV_BN 128        // narrow tiles (two workgroups per CU); 320-wide ones are picked by shape
#else
#define FP4Q_NV_BN 160
#endif
#endif
#ifndef FP4Q_NV_CB
#define FP4Q_NV_CB 64
#endif
#ifndef FP4Q_NV_NW
#define FP4Q_NV_NW 8
#endif
#ifndef FP4Q_NV_NS
#define FP4Q_NV_NS 2
#endif

inline int cdiv_i(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }


template <int FMT, int BM, int BN, int CB, int MINB, int NW, int NS, int M32 = 0>
hipError_t launch_mx3(const MxArgs& a0, hipStream_t s) {
  MxArgs a = a0;
  a.tiles_m = cdiv_i(a.M, BM);
  a.tiles_n = cdiv_i(a.N, BN);
  hipLaunchKernelGGL((k_gemm_mx3<FMT, BM, BN, CB, MINB, NW, NS, M32>), dim3((unsigned)(a.tiles_m * a.tiles_n)),
                     dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (!v) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* y,
                             int64_t ldy, hipStream_t s) {
  MxArgs p{a, as, b, bs, nullptr, nullptr, M, N, K, y, ldy, 0, 0};
  // K % 256 == 128 or tensors past 4 GiB: the register-staged kernel.
  if (K % (2 * FP4Q_MX_CB) || M * (K / 2) >= (int64_t(1) << 32) || N * (K / 2) >= (int64_t(1) << 32))
    return launch_gemm_mxfp4_staged(a, as, b, bs, M, N, K, y, ldy, s);
  // Column tile width by rounds of tiles over the compute units: a launch
  // takes ceil(tiles / CUs) rounds of one tile each, and a tile's time
  // grows with its width, so the width with the smaller rounds x width
  // wins (ties: 256).  For 2048 x 14336: 256 -> 448 tiles, 2 rounds x 256;
  // 224 -> 512 tiles, 2 rounds x 224 (measured 5% faster than 256-wide
  // tiles on the same 16 x 16 instructions, 2% faster than 256-wide tiles on
  // 32 x 32: 86.2 against 88.0 us).
  if constexpr (FP4Q_MX_BN == 256 && FP4Q_MX_CB == 128) {
    const int64_t cus = device_cus(), tm = cdiv_i(M, FP4Q_MX_BM);
    const int64_t c256 = cdiv_i(tm * cdiv_i(N, 256), cus) * 256;
    const int64_t c224 = cdiv_i(tm * cdiv_i(N, 224), cus) * 224;
    if (c224 < c256)
      return launch_mx3<FMT_MX, FP4Q_MX_BM, 224, FP4Q_MX_CB, FP4Q_MX_MINB, FP4Q_MX_NW, FP4Q_MX_NS, 0>(p, s);
  }
  return launch_mx3<FMT_MX, FP4Q_MX_BM, FP4Q_MX_BN, FP4Q_MX_CB, FP4Q_MX_MINB, FP4Q_MX_NW, FP4Q_MX_NS, FP4Q_MX_M32>(p, s);
}

// W4A16 runs on 32 x 32 x 16 bf16 instructions (the 16 x 16 x 32 shape
// sustains about half their rate): the looped core's 13 GEMMs 4% faster
// grouped (187.1 against 194.8 us) and 3% as single launches (256.7
// against 264.0 us, 256 x 64 tiles; 128 x 128: 281.3, 128 x 64: 267.7).
// Both forms keep the same K order per output, so a grouped launch equals
// single launches bit for bit.
#ifndef FP4Q_W16G_M32
#define FP4Q_W16G_M32 1
#endif
#ifndef FP4Q_W16M_M32
#define FP4Q_W16M_M32 1
#endif
#ifndef FP4Q_W16M_BM
#define FP4Q_W16M_BM 256      // single launches (16 x 16 form: 128 x 96 was the best of 64, 96, 128 wide)
#endif
#ifndef FP4Q_W16M_BN
#define FP4Q_W16M_BN 64
#endif
#ifndef FP4Q_W16M_CB
#define FP4Q_W16M_CB 64
#endif
#ifndef FP4Q_W16G_BM
#define FP4Q_W16G_BM 256      // grouped launches: many problems share the rounds, so larger tiles
#endif                        // fill the chip (looped-core step: 256 x 192 is 18% faster than 128 x 96,
#ifndef FP4Q_W16G_BN          // 7% faster than 256 x 128)
#define FP4Q_W16G_BN 192
#endif
#ifndef FP4Q_W16M_NW
#define FP4Q_W16M_NW 8
#endif

bool w4a16_direct_supported(int64_t lda, int64_t M, int64_t N, int64_t K) {
  return K % (2 * FP4Q_W16M_CB) == 0 && lda % 8 == 0 && M * lda * 2 < (int64_t(1) << 32) &&
         N * (K / 2) < (int64_t(1) << 32);
}

hipError_t launch_gemm_w4a16_direct(const void* a, int64_t lda, const uint8_t* b, const uint8_t* bs,
                                    const float* bts, int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                                    hipStream_t s) {
  MxArgs p{reinterpret_cast<const uint8_t*>(a), nullptr, b, bs, nullptr, bts, M, N, K, y, ldy, 0, 0, lda};
  return launch_mx3<FMT_W16, FP4Q_W16M_BM, FP4Q_W16M_BN, FP4Q_W16M_CB, 1, FP4Q_W16M_NW, 2, FP4Q_W16M_M32>(p, s);
}

hipError_t launch_gemm_w4a16_grouped(const fp4q_w4a16_problem* probs, int n, hipStream_t s) {
  // problems the direct-load kernel takes go into shared launches (longest
  // K first, so the longest tiles start first); the rest launch alone
  int idx[64];
  int nd = 0;
  for (int i = 0; i < n; ++i) {
    const fp4q_w4a16_problem& q = probs[i];
    if (w4a16_direct_supported(q.lda, q.M, q.N, q.K)) {
      idx[nd++] = i;
    } else {
      const hipError_t e = launch_gemm_w4a16(q.a_bf16, q.lda, q.b_codes, q.b_scales, q.b_tscale, q.M, q.N, q.K,
                                             q.y, q.ldy, s);
      if (e != hipSuccess) return e;
    }
  }
  for (int a = 1; a < nd; ++a)                     // stable insertion sort by K, descending
    for (int b = a; b > 0 && probs[idx[b]].K > probs[idx[b - 1]].K; --b) {
      const int t = idx[b]; idx[b] = idx[b - 1]; idx[b - 1] = t;
    }
  for (int base = 0; base < nd; base += kMaxGroup) {
    MxGroup g = {};
    g.n = (nd - base) < kMaxGroup ? (nd - base) : kMaxGroup;
    int wg = 0;
    for (int k = 0; k < g.n; ++k) {
      const fp4q_w4a16_problem& q = probs[idx[base + k]];
      MxArgs& a = g.prob[k];
      a = MxArgs{reinterpret_cast<const uint8_t*>(q.a_bf16), nullptr, q.b_codes, q.b_scales, nullptr, q.b_tscale,
                 q.M, q.N, q.K, q.y, q.ldy, cdiv_i(q.M, FP4Q_W16G_BM), cdiv_i(q.N, FP4Q_W16G_BN), q.lda};
      g.start[k] = wg;
      wg += a.tiles_m * a.tiles_n;
    }
    g.start[g.n] = wg;
    hipLaunchKernelGGL((k_gemm_mx3_grouped<FMT_W16, FP4Q_W16G_BM, FP4Q_W16G_BN, FP4Q_W16M_CB, 1, FP4Q_W16M_NW, 2, FP4Q_W16G_M32>),
                       dim3((unsigned)wg), dim3(FP4Q_W16M_NW * 64), 0, s, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* as, const float* ats,
                             const uint8_t* b, const uint8_t* bs, const float* bts, int64_t M,
                             int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s) {
  if (K % (2 * FP4Q_NV_CB) || M * (K / 2) >= (int64_t(1) << 32) || N * (K / 2) >= (int64_t(1) << 32))
    return launch_gemm_nvfp4_staged(a, as, ats, b, bs, bts, M, N, K, y, ldy, s);
  MxArgs p{a, as, b, bs, ats, bts, M, N, K, y, ldy, 0, 0};
#if FP4Q_NV_M32
  // Tile width by rounds: 128-wide tiles run two workgroups per CU, 320-wide
  // ones one (LDS); a round of either keeps a CU busy for about the same
  // width x workgroups, so the cost is rounds x that product, and the width
  // with the smaller cost wins (ties: 128).  4096 x 10240: 128 -> 1280 tiles,
  // 2.5 rounds of 512; 320 -> 512 tiles, exactly 2 rounds of 256 (7% faster).
  if constexpr (FP4Q_NV_BN == 128 && FP4Q_NV_BM == 256) {
    const int64_t cus = device_cus(), tm = cdiv_i(M, 256);
    const int64_t c128 = cdiv_i(tm * cdiv_i(N, 128), 2 * cus) * 256;
    const int64_t c320 = cdiv_i(tm * cdiv_i(N, 320), cus) * 320;
    if (c320 < c128) return launch_mx3<FMT_NV, 256, 320, FP4Q_NV_CB, 1, FP4Q_NV_NW, FP4Q_NV_NS, 1>(p, s);
  }
#endif
  return launch_mx3<FMT_NV, FP4Q_NV_BM, FP4Q_NV_BN, FP4Q_NV_CB, 1, FP4Q_NV_NW, FP4Q_NV_NS, FP4Q_NV_M32>(p, s);
}

}  // namespace fp4q
