// gemm.hip -- W4A4 and W4A16 GEMMs of libfp4q for gfx950 (CDNA4).
//
//   Y[M][N] = dequant(A)[M][K] * dequant(B)[N][K]^T, fp32 accumulate / output.
//
// MXFP4 ("MACaQ", core method: y = [(x*t)B]_MXFP4 W'^T_MXFP4): the packed
// E2M1 codes go straight into the block-scaled FP4 matrix core instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0 bytes as its per-lane,
// per-32-element scale operands -- the OCP MXFP4 block is exactly the
// instruction's scale block.
//
// NVFP4 ("Why Gated DeltaNet Survives 4-Bit Quantization", box "NVFP4 and
// W4A4"): the E4M3 scale belongs to a 16-element block and has a 3-bit
// mantissa, so it cannot ride the instruction's E8M0 scale.  Instead each
// element is dequantized EXACTLY to fp16 in registers: value(code) * 2^e
// with one v_cvt_scalef32_pk_f16_fp4 (the instruction applies the power of
// two), then times the scale mantissa (1 + f/8, or f for subnormal E4M3) with
// v_pk_mul_f16.  code * s_b has at most 2 + 4 significant bits and lies in
// [2^-10, 2688], so fp16 holds it exactly; the fp16 matrix core
// (v_mfma_f32_16x16x32_f16) multiplies exact values and accumulates in fp32.
// The two fp32 tensor scales are applied once in the epilogue.
//
// W4A16 (looped core: bf16 hidden state times the re-quantized weight): the
// weight is dequantized exactly to bf16 (fp32 value(code) * s_b, exact, then
// its upper half) and multiplied on the bf16 matrix core.
//
// Tiling (prefill kernels): 128 x 128 output tile per 256-thread workgroup,
// 2 x 2 wavefronts of 64 x 64, K staged 128 elements at a time through LDS
// with register double buffering.  Within a 128-element stage the 16 lanes
// of lane group g (= lane / 16) own elements [32g, 32g + 32) of their row,
// which is the FP4 instruction's own layout; the fp16 / bf16 instructions
// consume those 32 elements as four 8-element slices, one per instruction.
// A and B use the same assignment, so the dot product is unchanged.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.h"
#include "internal.h"

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// ------------------------------------------------------------ dequant ----

// E4M3 block scale split into a power of two (for the convert instruction)
// and an fp16 mantissa factor: s_b = pow2 * m exactly.
struct ScaleSplit {
  float pow2;
  v2h m;
};

__device__ __forceinline__ ScaleSplit split_e4m3(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, f = b & 7u;
  ScaleSplit s;
  if (e) {
    s.pow2 = __uint_as_float((e + 120u) << 23);                 // 2^(e-7)
    const _Float16 m = (_Float16)(1.0f + 0.125f * (float)f);     // exact
    s.m = v2h{m, m};
  } else {
    s.pow2 = __uint_as_float(118u << 23);                       // 2^-9
    const _Float16 m = (_Float16)(float)f;
    s.m = v2h{m, m};
  }
  return s;
}

// 8 codes (one dword, element 2i in the low nibble of byte i) -> 8 exact fp16.
__device__ __forceinline__ v8h dequant8_f16(uint32_t w, const ScaleSplit& s) {
  uint32_t o[4];
  o[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 0)) * s.m);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 1)) * s.m);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 2)) * s.m);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 3)) * s.m);
  return __builtin_bit_cast(v8h, uint4{o[0], o[1], o[2], o[3]});
}

// 8 codes -> 8 exact bf16: value(code) in fp32, times s_b (exact), upper half.
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

// ====================================================== prefill GEMMs ====
//
// One kernel template for the three prefill formats.  A 256-thread workgroup
// (2 x 2 wavefronts) owns a BM x BN output tile; each wavefront owns
// (BM/2) x (BN/2), i.e. FM x FN fragments of 16 x 16.  K advances one LDS
// stage at a time (register-staged double buffering, one barrier per
// stage).  LDS code rows are padded by 16 bytes, which makes the 16-byte
// fragment reads of eight consecutive rows land on disjoint banks.
//
// Tile order: the hardware hands workgroup b to XCD b % 8; each XCD is given
// a contiguous range of tile ids, walked in groups of GROUP_M row tiles so
// that the workgroups resident on one XCD share A rows and B columns in that
// XCD's L2.

enum Fmt { FMT_MX = 0, FMT_NV = 1, FMT_W16 = 2 };

struct GemmArgs {
  const uint8_t* A;       // codes [M][K/2] (MX, NV) or bf16 [M][lda] (W16)
  const uint8_t* As;      // A block scales (MX: [M][K/32], NV: [M][K/16]); unused for W16
  const float* Ats;       // A tensor scale (NV)
  const uint8_t* B;       // codes [N][K/2]
  const uint8_t* Bs;      // B block scales
  const float* Bts;       // B tensor scale (NV, W16)
  int64_t M, N, K, lda;
  float* Y;
  int64_t ldy;
  int tiles_m, tiles_n;
};

constexpr int GROUP_M = 8;

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<FMT_MX> {
  static constexpr int BK = 256;                  // K elements per stage
  static constexpr int SCB = BK / 32;             // scale bytes per row per stage
};
template <> struct FmtTraits<FMT_NV> {
  static constexpr int BK = 128;
  static constexpr int SCB = BK / 16;
};
template <> struct FmtTraits<FMT_W16> {
  static constexpr int BK = 128;
  static constexpr int SCB = BK / 16;
};

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  const int x = bid & 7, i = bid >> 3;
  const int base = nt >> 3, rem = nt & 7;
  const int t = x * base + (x < rem ? x : rem) + i;
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int in_g = t - group * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// Up to four scale bytes of one row from src (nullptr: none), little
// endian; bytes at or past the row end (`left` bytes remain in the row) are
// zero, so a K tail whose codes are zero also has zero scales: a stray
// E4M3 NaN byte of the next row would turn 0 x scale into NaN.
__device__ __forceinline__ uint32_t scale_word(const uint8_t* src, int64_t left, bool words) {
  if (!src) return 0u;
  if (words && left >= 4) return *reinterpret_cast<const uint32_t*>(src);
  uint32_t v = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (b < left) v |= (uint32_t)src[b] << (8 * b);
  return v;
}

template <int FMT, int BM, int BN, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void k_gemm(const GemmArgs p) {
  using T = FmtTraits<FMT>;
  constexpr int BK = T::BK, SCB = T::SCB;
  constexpr int CB = BK / 2;                                 // code bytes per row per stage
  constexpr int LDC = CB + 16;                               // padded code row (bytes)
  constexpr int ARB = (FMT == FMT_W16) ? BK * 2 : CB;        // A bytes per row per stage
  constexpr int LDAR = ARB + 16;                             // padded A row (bytes)
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int A_CH = BM * ARB / 16, B_CH = BN * CB / 16;   // 16-byte chunks per stage
  constexpr int A_LD = (A_CH + kThreads - 1) / kThreads, B_LD = (B_CH + kThreads - 1) / kThreads;
  constexpr int A_SC = (FMT == FMT_W16) ? 0 : BM;            // scale rows staged per stage
  constexpr int SC_ROWS = A_SC + BN;
  constexpr int SCW = SCB / 4;                               // scale words per row per stage
  constexpr int SC_LD = (SC_ROWS * SCW + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) uint8_t lA[2][BM * LDAR];
  __shared__ __attribute__((aligned(16))) uint8_t lB[2][BN * LDC];
  __shared__ uint32_t lS[2][SC_ROWS * SCW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 4, r16 = lane & 15;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t ldb = p.K / 2, lds = p.K / (FMT == FMT_MX ? 32 : 16);
  const int KT = (int)((p.K + BK - 1) / BK);   // the last stage may be partly empty (K % 32 == 0 only)
  // scale rows are whole 4-byte words when K / 32 (MXFP4) or K / 16 is a
  // multiple of 4; otherwise they are read byte by byte
  const bool words = (lds & 3) == 0;

  uint4 ra[A_LD], rb[B_LD];
  uint32_t rs[SC_LD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + kThreads * i;
      constexpr int CPR = ARB / 16;
      const int64_t r = m0 + c / CPR;
      uint4 v = {0u, 0u, 0u, 0u};
      const int64_t kb = (int64_t)kt * ARB + (c % CPR) * 16;    // byte offset within the row
      if (c < A_CH && r < p.M && kb < (FMT == FMT_W16 ? p.K * 2 : ldb)) {
        if constexpr (FMT == FMT_W16)
          v = *reinterpret_cast<const uint4*>(p.A + (r * p.lda + (int64_t)kt * BK) * 2 + (c % CPR) * 16);
        else
          v = *reinterpret_cast<const uint4*>(p.A + r * ldb + (int64_t)kt * CB + (c % CPR) * 16);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + kThreads * i;
      constexpr int CPR = CB / 16;
      const int64_t r = n0 + c / CPR;
      uint4 v = {0u, 0u, 0u, 0u};
      const int64_t kb = (int64_t)kt * CB + (c % CPR) * 16;
      if (c < B_CH && r < p.N && kb < ldb) v = *reinterpret_cast<const uint4*>(p.B + r * ldb + kb);
      rb[i] = v;
    }
#pragma unroll
    for (int i = 0; i < SC_LD; ++i) {
      const int c = tid + kThreads * i;            // (row, word) of the staged scales
      const int row = c / SCW, w = c % SCW;
      const int64_t kb = (int64_t)kt * SCB + 4 * w;
      const uint8_t* src = nullptr;
      if (row < A_SC) {
        const int64_t r = m0 + row;
        if (r < p.M && kb < lds) src = p.As + r * lds + kb;
      } else if (row < SC_ROWS) {
        const int64_t r = n0 + (row - A_SC);
        if (r < p.N && kb < lds) src = p.Bs + r * lds + kb;
      }
      rs[i] = scale_word(src, lds - kb, words);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + kThreads * i;
      constexpr int CPR = ARB / 16;
      if (c < A_CH) *reinterpret_cast<uint4*>(&lA[buf][(c / CPR) * LDAR + (c % CPR) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + kThreads * i;
      constexpr int CPR = CB / 16;
      if (c < B_CH) *reinterpret_cast<uint4*>(&lB[buf][(c / CPR) * LDC + (c % CPR) * 16]) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < SC_LD; ++i) {
      const int c = tid + kThreads * i;
      if (c < SC_ROWS * SCW) lS[buf][c] = rs[i];
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* la = lA[buf];
    const uint8_t* lb = lB[buf];
    if constexpr (FMT == FMT_MX) {
      // two 128-element instruction steps per stage; lane group g owns
      // bytes [16 g, 16 g + 16) of each 64-byte half
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i af[FM];
        int sa[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * (BM / 2) + i * 16 + r16;
          const uint4 q = *reinterpret_cast<const uint4*>(la + row * LDAR + ks * 64 + g * 16);
          af[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          sa[i] = (int)((reinterpret_cast<const uint8_t*>(&lS[buf][row * SCW]))[ks * 4 + g]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * (BN / 2) + j * 16 + r16;
          const uint4 q = *reinterpret_cast<const uint4*>(lb + row * LDC + ks * 64 + g * 16);
          const v8i bf = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
          const int sb = (int)((reinterpret_cast<const uint8_t*>(&lS[buf][(A_SC + row) * SCW]))[ks * 4 + g]);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[i][j], 4, 4, 0, sa[i], 0, sb);
        }
      }
    } else {
      // lane group g owns elements [32 g, 32 g + 32) of the stage: two
      // NVFP4 blocks (h = 0, 1), each consumed as two 8-element slices
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 qa[FM];
        ScaleSplit xa[FM];
        if constexpr (FMT == FMT_NV) {
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int row = wm * (BM / 2) + i * 16 + r16;
            qa[i] = *reinterpret_cast<const uint2*>(la + row * LDAR + g * 16 + h * 8);
            xa[i] = split_e4m3((reinterpret_cast<const uint8_t*>(&lS[buf][row * SCW]))[2 * g + h]);
          }
        }
        uint2 qb[FN];
        ScaleSplit xb[FN];
        float sbf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * (BN / 2) + j * 16 + r16;
          qb[j] = *reinterpret_cast<const uint2*>(lb + row * LDC + g * 16 + h * 8);
          const uint32_t sbyte = (reinterpret_cast<const uint8_t*>(&lS[buf][(A_SC + row) * SCW]))[2 * g + h];
          if constexpr (FMT == FMT_NV) xb[j] = split_e4m3(sbyte);
          else sbf[j] = e4m3_decode(sbyte);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if constexpr (FMT == FMT_NV) {
            v8h ha[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) ha[i] = dequant8_f16(s2 ? qa[i].y : qa[i].x, xa[i]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const v8h hb = dequant8_f16(s2 ? qb[j].y : qb[j].x, xb[j]);
#pragma unroll
              for (int i = 0; i < FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[i], hb, acc[i][j], 0, 0, 0);
            }
          } else {
            const int s = 2 * h + s2;
            v8bf ha[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              const int row = wm * (BM / 2) + i * 16 + r16;
              ha[i] = *reinterpret_cast<const v8bf*>(la + row * LDAR + (32 * g + 8 * s) * 2);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const v8bf hb = dequant8_bf16(s2 ? qb[j].y : qb[j].x, sbf[j]);
#pragma unroll
              for (int i = 0; i < FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[i], hb, acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  float tsc = 1.0f;
  if constexpr (FMT == FMT_NV) tsc = (*p.Ats) * (*p.Bts);
  if constexpr (FMT == FMT_W16) tsc = *p.Bts;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + i * 16 + g * 4 + r;
        const int64_t col = n0 + wn * (BN / 2) + j * 16 + r16;
        if (row < p.M && col < p.N) {
          float v = acc[i][j][r];
          if constexpr (FMT != FMT_MX) v = v * tsc;
          p.Y[row * p.ldy + col] = v;
        }
      }
}

}  // namespace

// Tile shapes (BM, BN, minimum workgroups per CU) of the prefill kernels.
#ifndef FP4Q_MX_TILE
#define FP4Q_MX_TILE 128, 224, 1
#endif
#ifndef FP4Q_NV_TILE
#define FP4Q_NV_TILE 128, 256, 1
#endif
#ifndef FP4Q_W16_TILE
#define FP4Q_W16_TILE 128, 64, 4     // small tiles: the looped core has N, K in {768, 3072} (measured)
#endif

namespace {
template <int FMT, int BM, int BN, int MINB>
hipError_t launch_tiled(const GemmArgs& a0, hipStream_t s) {
  GemmArgs a = a0;
  a.tiles_m = (int)cdiv(a.M, BM);
  a.tiles_n = (int)cdiv(a.N, BN);
  hipLaunchKernelGGL((k_gemm<FMT, BM, BN, MINB>), dim3((unsigned)a.tiles_m * a.tiles_n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_mxfp4_staged(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                    const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* y,
                                    int64_t ldy, hipStream_t s) {
  GemmArgs p{a, as, nullptr, b, bs, nullptr, M, N, K, 0, y, ldy, 0, 0};
  return launch_tiled<FMT_MX, FP4Q_MX_TILE>(p, s);
}

hipError_t launch_gemm_nvfp4_staged(const uint8_t* a, const uint8_t* as, const float* ats,
                             const uint8_t* b, const uint8_t* bs, const float* bts, int64_t M,
                             int64_t N, int64_t K, float* y, int64_t ldy, hipStream_t s) {
  GemmArgs p{a, as, ats, b, bs, bts, M, N, K, 0, y, ldy, 0, 0};
  return launch_tiled<FMT_NV, FP4Q_NV_TILE>(p, s);
}

hipError_t launch_gemm_w4a16(const void* a, int64_t lda, const uint8_t* b, const uint8_t* bs,
                             const float* bts, int64_t M, int64_t N, int64_t K, float* y,
                             int64_t ldy, hipStream_t s) {
#ifndef FP4Q_W16_STAGED_ONLY
  if (w4a16_direct_supported(lda, M, N, K)) return launch_gemm_w4a16_direct(a, lda, b, bs, bts, M, N, K, y, ldy, s);
#endif
  GemmArgs p{reinterpret_cast<const uint8_t*>(a), nullptr, nullptr, b, bs, bts, M, N, K, lda, y, ldy, 0, 0};
  return launch_tiled<FMT_W16, FP4Q_W16_TILE>(p, s);
}

}  // namespace fp4q
