// gemm_decode.hip -- decode-shaped NVFP4 W4A4 GEMM (M <= 16) for gfx950,
// with the activation quantization optionally fused into the prologue
// ("Why Gated DeltaNet Survives 4-Bit Quantization", limitations: decode was
// slowed by the separate small-batch NVFP4 activation-quantization kernel).
//
// The weight (N x K NVFP4, ~50 MB for 17408 x 5120) is read exactly once, so
// each form is an HBM stream with as little work per weight byte as
// possible.  Three forms, picked by shape:
//  * M = 1: row streaming (k_decode_rows) -- each wavefront walks whole
//    weight rows with coalesced 1 KiB loads and v_dot2 against the
//    activation held as exact fp16 in LDS;
//  * 2 <= M <= 16, K <= 5120, K % 256 == 0: the streamed form
//    (k_decode_stream) -- 16-row weight groups pulled whole into LDS by
//    direct global->LDS loads, sixteen wavefronts splitting K on the fp16
//    matrix core with register-resident activation fragments;
//  * other shapes: the register-staged form (k_decode) -- 64 weight rows per
//    workgroup, K streamed through registers.
// Every form dequantizes both operands exactly to fp16 (code * s_b has at
// most 6 significant bits), accumulates in fp32, adds partial sums in a
// fixed order (so the fused and the pre-quantized entry points agree bit for
// bit) and applies the two tensor scales once at the end.  The fused
// prologues quantize with exactly the fp4q_quantize_nvfp4 recipe; with a
// dynamic activation scale the rows and streamed forms derive it from the
// exact amax in every workgroup (max is order-free), the register-staged
// form reads it from a separate amax pass.

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "codec.h"
#include "internal.h"

namespace fp4q {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int RPW = 32;                 // weight rows per wavefront
constexpr int FRAGS = RPW / 16;         // 16-row fragments per wavefront
constexpr int RPG = 2 * RPW;            // weight rows per workgroup (2 row groups x 2 K halves)
constexpr int PF = 4;                   // stages in flight per register set
constexpr int SK_MAXK = 7168;           // A codes + scales (~9 K bytes + padding) within 64 KiB of LDS
constexpr uint32_t kAmaxFlag = 0x80000000u;

typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront in a fixed order: pairs, quads,
// half-rows (row_half_mirror), rows of 16 (row_mirror), then the four row
// sums.  Every lane receives the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Two E4M3 block scales (low 16 bits of w) -> fp16, each splatted to both
// halves.  Every E4M3 value is exactly an fp16 normal.
__device__ __forceinline__ void e4m3x2_to_h2(uint32_t w, v2h& s0, v2h& s1) {
  const v2h t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  s0 = v2h{t[0], t[0]};
  s1 = v2h{t[1], t[1]};
}

__device__ __forceinline__ v8h dequant8(uint32_t w, v2h sb) {
  const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * sb);
  const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * sb);
  const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * sb);
  const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * sb);
  return __builtin_bit_cast(v8h, uint4{o0, o1, o2, o3});
}

struct Stage {                            // one wavefront's weight data of PF stages
  uint4 q[PF][FRAGS];
  uint32_t s[PF][FRAGS];                  // two E4M3 bytes (blocks 2g, 2g+1)
};

template <bool FUSED>
__global__ __launch_bounds__(kThreads) void k_decode(
    const uint16_t* __restrict__ Abf, int64_t lda, const uint8_t* __restrict__ Ac,
    const uint8_t* __restrict__ As, float* Ats, int a_dynamic, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ Bts, int64_t M, int64_t N, int64_t K,
    float* __restrict__ Y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int64_t ldb = K / 2, lds = K / 16;
  const int64_t lrow = ldb + 16, lsrow = lds + 4;     // padded LDS row strides (bytes)
  uint8_t* lAc = smem;                                // [16][lrow]
  uint8_t* lAs = smem + 16 * lrow;                    // [16][lsrow]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int rg = wave & 1, kh = wave >> 1;            // row group, K half
  // K stages of 128; with K % 128 != 0 the last one is partly empty: lane
  // group g of stage kt holds 32-element block 4 kt + g, present while it is
  // below K / 32, and absent blocks contribute zero codes and zero scales
  const int KT = (int)((K + 127) / 128), nblk = (int)(K / 32);
  const int kt_begin = kh ? KT / 2 : 0, kt_end = kh ? KT : KT / 2;

  // weight rows of this lane (one per fragment), clamped into the tensor
  const uint8_t* brow[FRAGS];
  const uint8_t* bsrow[FRAGS];
  const int64_t wrow0 = (int64_t)blockIdx.x * RPG + rg * RPW;
#pragma unroll
  for (int f = 0; f < FRAGS; ++f) {
    int64_t r = wrow0 + f * 16 + r16;
    r = r < N ? r : N - 1;
    brow[f] = B + r * ldb + g * 16;
    bsrow[f] = Bs + r * lds + 2 * g;
  }
  auto load_group = [&](Stage& st, int kt0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int kt = kt0 + p;
#pragma unroll
      for (int f = 0; f < FRAGS; ++f) {
        if (kt < kt_end && 4 * kt + g < nblk) {
          const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(brow[f] + (int64_t)kt * 64));
          st.q[p][f] = uint4{q[0], q[1], q[2], q[3]};
          st.s[p][f] = *reinterpret_cast<const uint16_t*>(bsrow[f] + (int64_t)kt * 8);
        } else {
          st.q[p][f] = uint4{0u, 0u, 0u, 0u};
          st.s[p][f] = 0u;
        }
      }
    }
  };

  Stage cur, nxt;
  load_group(cur, kt_begin);              // weight stream starts before the prologue

  // ---- prologue: activation rows [0, M) into LDS, rows [M, 16) zero
  // (all index arithmetic fits 32 bits: K <= 7168, M <= 16)
  float ats;
  const int Ki = (int)K, Mi = (int)M;
  const int lrow_i = (int)lrow, lsrow_i = (int)lsrow, ldb_i = (int)ldb, lds_i = (int)lds;
  const int cpr16 = Ki / 32;                          // 16-byte code chunks per row
  for (int c = tid; c < (16 - Mi) * cpr16; c += kThreads) {
    const int r = Mi + c / cpr16, cc = c % cpr16;
    *reinterpret_cast<uint4*>(lAc + r * lrow_i + cc * 16) = uint4{0u, 0u, 0u, 0u};
  }
  for (int c = tid; c < (16 - Mi) * lds_i; c += kThreads) {
    const int r = Mi + c / lds_i;
    lAs[r * lsrow_i + c % lds_i] = 0;
  }
  if constexpr (FUSED) {
    // quantize A[0:M) exactly as k_quant_nvfp4 does (one lane per 8 values,
    // lane pairs share a 16-block); loads are issued four at a time
    const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(Ats));
    ats = (a_dynamic && (u & kAmaxFlag)) ? __uint_as_float(u & 0x7FFFFFFFu) / 1536.0f : __uint_as_float(u);
    const float six_st = 6.0f * ats;
    const int cpr = Ki / 8, nch = Mi * cpr;
    const int nch_pad = (nch + 4 * kThreads - 1) / (4 * kThreads) * (4 * kThreads);  // all lanes join the DPP
    for (int c0 = tid; c0 < nch_pad; c0 += 4 * kThreads) {
      uint4 q[4];
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int c = c0 + u4 * kThreads;
        q[u4] = c < nch ? *reinterpret_cast<const uint4*>(Abf + (int64_t)(c / cpr) * lda + (c % cpr) * 8)
                        : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int c = c0 + u4 * kThreads;
        const uint32_t w[4] = {q[u4].x, q[u4].y, q[u4].z, q[u4].w};
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
        a = fmaxf(a, dpp_xor1(a));
        uint32_t sb = 0;
        if (a > 0.0f && ats > 0.0f) sb = e4m3_ceil(a / six_st);
        const float sc = ats * e4m3_decode(sb);
        const float rho = 1.0f / sc;
        uint32_t p = 0;
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0] * rho, v[1] * rho, 1.0f, 0);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * rho, v[3] * rho, 1.0f, 1);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * rho, v[5] * rho, 1.0f, 2);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * rho, v[7] * rho, 1.0f, 3);
        if (c < nch) {
          const int r = c / cpr, c8 = c % cpr;
          *reinterpret_cast<uint32_t*>(lAc + r * lrow_i + c8 * 4) = (sc == 0.0f) ? 0u : p;
          if (!(c & 1)) lAs[r * lsrow_i + (c8 >> 1)] = (uint8_t)sb;
        }
      }
    }
    if (a_dynamic && blockIdx.x == 0 && tid == 0) *Ats = ats;
  } else {
    ats = *Ats;
    for (int c0 = tid; c0 < Mi * cpr16; c0 += 4 * kThreads) {
      uint4 q[4];
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int c = c0 + u4 * kThreads;
        q[u4] = c < Mi * cpr16 ? *reinterpret_cast<const uint4*>(Ac + (int64_t)(c / cpr16) * ldb_i + (c % cpr16) * 16)
                               : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        const int c = c0 + u4 * kThreads;
        if (c < Mi * cpr16) *reinterpret_cast<uint4*>(lAc + (c / cpr16) * lrow_i + (c % cpr16) * 16) = q[u4];
      }
    }
    for (int c = tid; c < Mi * lds_i; c += kThreads) lAs[(c / lds_i) * lsrow_i + c % lds_i] = As[c];
  }
  __syncthreads();

  v4f acc[FRAGS];
#pragma unroll
  for (int f = 0; f < FRAGS; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& st, int kt0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int kt = kt0 + p;
      if (kt < kt_end) {
        // A: lane group g owns elements [32 g, 32 g + 32) of the stage
        const bool va = 4 * kt + g < nblk;
        const uint4 qa = va ? *reinterpret_cast<const uint4*>(lAc + r16 * lrow + (int64_t)kt * 64 + g * 16)
                            : uint4{0u, 0u, 0u, 0u};
        const uint32_t wsa = va ? *reinterpret_cast<const uint16_t*>(lAs + r16 * lsrow + (int64_t)kt * 8 + 2 * g) : 0u;
        v2h sa0, sa1;
        e4m3x2_to_h2(wsa, sa0, sa1);
        v2h sb[FRAGS][2];
#pragma unroll
        for (int f = 0; f < FRAGS; ++f) e4m3x2_to_h2(st.s[p][f], sb[f][0], sb[f][1]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t wa = s == 0 ? qa.x : s == 1 ? qa.y : s == 2 ? qa.z : qa.w;
          const v8h ha = dequant8(wa, s < 2 ? sa0 : sa1);
#pragma unroll
          for (int f = 0; f < FRAGS; ++f) {
            const uint4& qb = st.q[p][f];
            const uint32_t wb = s == 0 ? qb.x : s == 1 ? qb.y : s == 2 ? qb.z : qb.w;
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, dequant8(wb, sb[f][s >> 1]), acc[f], 0, 0, 0);
          }
        }
      }
    }
  };
  // two register sets in strict alternation: the loads of one set are in
  // flight while the other is consumed
  for (int kt0 = kt_begin; kt0 < kt_end; kt0 += 2 * PF) {
    if (kt0 + PF < kt_end) load_group(nxt, kt0 + PF);
    compute(cur, kt0);
    if (kt0 + 2 * PF < kt_end) load_group(cur, kt0 + 2 * PF);
    if (kt0 + PF < kt_end) compute(nxt, kt0 + PF);
  }

  // ---- K-half reduction (fixed order: first half + second half) and store.
  // lane (r16, g) holds rows m = 4 g + r of output columns wrow0 + 16 f + r16
  __syncthreads();                                    // activation tiles no longer read
  float* red = reinterpret_cast<float*>(smem);        // [2 row groups][FRAGS][4][64]
  if (kh == 1) {
#pragma unroll
    for (int f = 0; f < FRAGS; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((rg * FRAGS + f) * 4 + r) * 64 + lane] = acc[f][r];
  }
  __syncthreads();
  if (kh == 0) {
    const float tsc = ats * (*Bts);
#pragma unroll
    for (int f = 0; f < FRAGS; ++f) {
      const int64_t n = wrow0 + f * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = g * 4 + r;
        const float v = acc[f][r] + red[((rg * FRAGS + f) * 4 + r) * 64 + lane];
        if (m < M && n < N) Y[m * ldy + n] = v * tsc;
      }
    }
  }
}

// Quantizes the M x K bf16 activation rows with the NVFP4 recipe of
// fp4q_quantize_nvfp4, using all NT threads of the workgroup: every thread
// loads its (at most U) 8-element chunks once (chunk c: row c / (K / 8),
// elements [8 (c % (K / 8)), +8)); with `dynamic` the tensor scale is
// fl(amax / 1536) over the whole activation (max is exact, so every
// workgroup derives the same value), else ats_in.  Lane pairs share a
// 16-block (DPP); put(r, c8, codes, scale) stores one chunk's four code
// bytes and, on even c8, the block scale.  PAIRED: each lane of a pair
// computes the block scales of one of two chunks and passes them to the
// other, and chunk rows and columns advance without a division per chunk
// (fewer instructions, more live registers).  Returns the tensor scale.
template <int NT, int U, bool PAIRED, typename Put>
__device__ __forceinline__ float quantize_act_block(const uint16_t* __restrict__ A, int64_t lda, int M, int K,
                                                    float ats_in, bool dynamic, float* red, Put put) {
  const int tid = threadIdx.x, cpr = K / 8, nch = M * cpr;
  // row and column of chunk tid + u NT: one division per thread, then
  // steps of NT chunks (q_nt rows and r_nt < cpr columns: at most one wrap)
  const int q_nt = NT / cpr, r_nt = NT - q_nt * cpr;      // uniform
  const int row0 = tid / cpr, col0 = tid - row0 * cpr;
  auto advance = [&](int& row, int& col) {
    row += q_nt;
    col += r_nt;
    if (col >= cpr) {
      col -= cpr;
      ++row;
    }
  };
  uint4 q[U];
  if constexpr (PAIRED) {
    int row = row0, col = col0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = tid + u * NT < nch;                  // else chunk 0, real data: harmless to the max
      q[u] = *reinterpret_cast<const uint4*>(A + (in ? (int64_t)row * lda + col * 8 : 0));
      advance(row, col);
    }
  } else {                                                 // fewer live registers: a division per chunk
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + u * NT;
      const int cc = c < nch ? c : 0;
      q[u] = *reinterpret_cast<const uint4*>(A + (int64_t)(cc / cpr) * lda + (cc % cpr) * 8);
    }
  }
  float ats = ats_in;
  if (dynamic) {
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a = fmaxf(a, fmaxf(__builtin_fabsf(__uint_as_float(w[i] << 16)), __builtin_fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    if ((tid & 63) == 0) red[tid >> 6] = a;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t = fmaxf(t, red[w]);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    ats = t / 1536.0f;
  }
  const float six_st = 6.0f * ats;
  // Chunks u and u + 1 at a time: the block maxima of both, then the even
  // lane of a pair computes the block scales of u and the odd lane those of
  // u + 1, and each passes its results to the other (an odd U's last chunk
  // is done by both lanes).
  auto unpack = [&](const uint4& qq, float v[8]) {
    const uint32_t w[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  };
  auto block_max = [&](const float v[8]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
    return fmaxf(a, dpp_xor1(a));                          // cpr is even: pairs share a row
  };
  auto scales_of = [&](float a, uint32_t& sb, float& sc, float& rho) {
    sb = 0;
    if (a > 0.0f && ats > 0.0f) sb = e4m3_ceil(a / six_st);
    sc = ats * e4m3_decode(sb);
    rho = 1.0f / sc;
  };
  // emits chunks in increasing u, walking the same rows and columns again
  int erow = row0, ecol = col0;
  auto emit = [&](int u, const float v[8], uint32_t sb, float sc, float rho) {
    const int c = tid + u * NT;
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0] * rho, v[1] * rho, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * rho, v[3] * rho, 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * rho, v[5] * rho, 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * rho, v[7] * rho, 1.0f, 3);
    if constexpr (PAIRED) {
      if (c < nch) put(erow, ecol, (sc == 0.0f) ? 0u : p, sb);
      advance(erow, ecol);
    } else {
      if (c < nch) put(c / cpr, c % cpr, (sc == 0.0f) ? 0u : p, sb);
    }
  };
  if constexpr (!PAIRED) {                                // fewer live registers: both lanes do all
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[8];
      unpack(q[u], v);
      uint32_t sb;
      float sc, rho;
      scales_of(block_max(v), sb, sc, rho);
      emit(u, v, sb, sc, rho);
    }
    return ats;
  }
  const bool odd = tid & 1;
#pragma unroll
  for (int u = 0; u + 1 < U; u += 2) {
    float v0[8], v1[8];
    unpack(q[u], v0);
    unpack(q[u + 1], v1);
    const float a0 = block_max(v0), a1 = block_max(v1);
    uint32_t sb;
    float sc, rho;
    scales_of(odd ? a1 : a0, sb, sc, rho);
    const uint32_t sbp = (uint32_t)__float_as_int(dpp_xor1(__int_as_float((int)sb)));
    const float scp = dpp_xor1(sc), rhop = dpp_xor1(rho);
    emit(u, v0, odd ? sbp : sb, odd ? scp : sc, odd ? rhop : rho);
    emit(u + 1, v1, odd ? sb : sbp, odd ? sc : scp, odd ? rho : rhop);
  }
  if constexpr (U % 2 == 1) {
    float v[8];
    unpack(q[U - 1], v);
    uint32_t sb;
    float sc, rho;
    scales_of(block_max(v), sb, sc, rho);
    emit(U - 1, v, sb, sc, rho);
  }
  return ats;
}

// ------------------------------------------------------------ M <= 4 ----
//
// Row-streaming form for the smallest batches: each wavefront walks whole
// weight rows (the 2.5 KiB of codes of a 5120-wide row are read as 1 KiB
// contiguous wavefront loads), and adjacent wavefronts take adjacent rows,
// so the chip sweeps the weight front to back -- on this memory system a
// contiguous sweep streams ~2.2x faster than the row-strided fragment
// pattern of the matrix-core kernel.  Lane l owns 16-byte chunks
// l, l + 64, l + 128, ... of the row (32 K elements each).  The activation
// rows are held in LDS already dequantized to fp16 (exact); each 16-element
// weight block is multiplied with v_dot2 on its raw code values and the
// block sum is scaled by the weight's E4M3 factor in fp32; a fixed-order
// wavefront reduction finishes each output.
constexpr int kRowsMaxM = 4;
#ifndef FP4Q_ROWS_GRID
#define FP4Q_ROWS_GRID 512   // two 4-wavefront workgroups per CU (measured at M = 1, K = 5120: 9% faster
                             // than three, 11% faster than four; one is within 1% of two)
#endif

template <int CH>
struct RowData {                                        // one wavefront's share of one weight row
  uint4 q[CH];                                          // 16-byte code chunks lane + 64 j
  uint32_t s[CH];                                       // their two E4M3 block scales
};

// CH = 16-byte code chunks per lane (ceil(K / 32 / 64)).  Every load is
// issued unconditionally from a clamped, in-bounds address so that the
// number of loads in flight is the same on every path and the waits for a
// row never have to drain the loads of the rows behind it.
template <bool FUSED, int CH, int MM>
__global__ __launch_bounds__(kThreads) void k_decode_rows(
    const uint16_t* __restrict__ Abf, int64_t lda, const uint8_t* __restrict__ Ac,
    const uint8_t* __restrict__ As, float* Ats, int a_dynamic, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ Bts, int64_t M, int64_t N, int64_t K,
    float* __restrict__ Y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  _Float16* lA = reinterpret_cast<_Float16*>(smem);     // [M][K] exact fp16 activation values
  const int tid = threadIdx.x, lane = tid & 63;
  const int Ki = (int)K, Mi = MM, ldb = Ki / 2, lds = Ki / 16;
  const int nchunk = Ki / 32;                           // 16-byte code chunks per row

  // ---- weight row stream: wavefront w of the grid takes rows w, w + W, ...
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wv = (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(tid >> 6);
  int cj[CH];                                           // this lane's chunk index, clamped
  bool cvalid[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    cvalid[j] = c < nchunk;
    cj[j] = cvalid[j] ? c : nchunk - 1;
  }
  auto load_row = [&](RowData<CH>& d, int64_t n) {
    n = n < N ? n : N - 1;
    const uint8_t* br = B + n * ldb;
    const uint8_t* sr = Bs + n * lds;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(br + cj[j] * 16));
      d.q[j] = uint4{q[0], q[1], q[2], q[3]};
      d.s[j] = *reinterpret_cast<const uint16_t*>(sr + 2 * cj[j]);
    }
  };
  RowData<CH> r0, r1, r2;                               // rotate with static indices
  load_row(r0, wv);                                     // the stream starts before the prologue
  __builtin_amdgcn_sched_barrier(0);
  load_row(r1, wv + nwaves);
  __builtin_amdgcn_sched_barrier(0);
  load_row(r2, wv + 2 * nwaves);
  __builtin_amdgcn_sched_barrier(0);

  // ---- activation -> fp16 in LDS (codes decoded and multiplied by s_b)
  float ats;
  auto put8 = [&](int r, int c8, uint32_t p, uint32_t sb) {
    const v2h t = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false));
    const v2h s2 = v2h{t[0], t[0]};
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 0)) * s2);
    o.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 1)) * s2);
    o.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 2)) * s2);
    o.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 3)) * s2);
    *reinterpret_cast<uint4*>(lA + r * Ki + c8 * 8) = o;
  };
  const int cpr = Ki / 8, nch = Mi * cpr;
  __shared__ float red_amax[kThreads / 64];
  if constexpr (FUSED) {
    // paired scales for the one-row form (2% faster; the multi-row forms
    // would pay more registers than the scales save)
    ats = quantize_act_block<kThreads, 4 * MM, MM == 1>(Abf, lda, Mi, Ki, *Ats, a_dynamic != 0, red_amax,
                                               [&](int r, int c8, uint32_t p, uint32_t sb) { put8(r, c8, p, sb); });
    if (a_dynamic && blockIdx.x == 0 && tid == 0) *Ats = ats;
  } else {
    ats = *Ats;
    for (int c = tid; c < nch; c += kThreads) {
      const int r = c / cpr, c8 = c % cpr;
      put8(r, c8, *reinterpret_cast<const uint32_t*>(Ac + (int64_t)r * ldb + c8 * 4), As[(int64_t)r * lds + (c8 >> 1)]);
    }
  }
  // LDS writes complete, then the barrier; the weight loads stay in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const float tsc = ats * (*Bts);
  // one activation row: this lane's chunks are the same in every weight row,
  // so their 32 fp16 values per chunk stay in registers for the whole stream
  // (no LDS reads in the row loop; measured 4% faster at M = 1)
  uint4 areg[MM == 1 ? CH : 1][4];
  if constexpr (MM == 1) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) areg[j][q] = reinterpret_cast<const uint4*>(lA + cj[j] * 32)[q];
  }
  auto process_row = [&](const RowData<CH>& cur, int64_t n) {
    float acc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t w4[4] = {cur.q[j].x, cur.q[j].y, cur.q[j].z, cur.q[j].w};
      // a lane past the end of the row contributes zero through its scales
      const v2f sbv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cur.s[j], 1.0f, false);
      const float sb0 = cvalid[j] ? sbv[0] : 0.0f;
      const float sb1 = cvalid[j] ? sbv[1] : 0.0f;
      v2h wq[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wq[4 * i + 0] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[i], 1.0f, 0));
        wq[4 * i + 1] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[i], 1.0f, 1));
        wq[4 * i + 2] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[i], 1.0f, 2));
        wq[4 * i + 3] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w4[i], 1.0f, 3));
      }
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const uint4* ap = reinterpret_cast<const uint4*>(lA + m * Ki + cj[j] * 32);
        float bs[2] = {0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 a0 = MM == 1 ? areg[MM == 1 ? j : 0][2 * h] : ap[2 * h];
          const uint4 a1 = MM == 1 ? areg[MM == 1 ? j : 0][2 * h + 1] : ap[2 * h + 1];
          const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bs[h] = __builtin_amdgcn_fdot2(wq[8 * h + e], __builtin_bit_cast(v2h, av[e]), bs[h], false);
        }
        acc[m] = acc[m] + bs[0] * sb0;
        acc[m] = acc[m] + bs[1] * sb1;
      }
    }
    // lane l stores output l % MM (lanes with the same output store the
    // same value); an unconditional store keeps the wait counts exact
    float out = 0.0f;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float v = wave_sum(acc[m]) * tsc;
      out = (lane % MM == m) ? v : out;
    }
    Y[(lane % MM) * ldy + n] = out;
  };
  // the scheduling barriers keep each refill behind the row it replaces, so
  // the loads stay in issue order and each wait covers exactly one row
  // (the refills are unconditional: past the end they re-read the last row)
  for (int64_t n = wv; n < N; n += 3 * nwaves) {
    process_row(r0, n);
    __builtin_amdgcn_sched_barrier(0);
    load_row(r0, n + 3 * nwaves);
    __builtin_amdgcn_sched_barrier(0);
    if (n + nwaves < N) process_row(r1, n + nwaves);
    __builtin_amdgcn_sched_barrier(0);
    load_row(r1, n + 4 * nwaves);
    __builtin_amdgcn_sched_barrier(0);
    if (n + 2 * nwaves < N) process_row(r2, n + 2 * nwaves);
    __builtin_amdgcn_sched_barrier(0);
    load_row(r2, n + 5 * nwaves);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool FUSED>
hipError_t launch_rows(int ch, unsigned grid, size_t shm, hipStream_t s, const uint16_t* abf, int64_t lda,
                       const uint8_t* ac, const uint8_t* as, float* ats, int dyn, const uint8_t* b,
                       const uint8_t* bs, const float* bts, int64_t M, int64_t N, int64_t K, float* y,
                       int64_t ldy) {
#define FP4Q_ROWS_CASE(C, MC)                                                                          \
  case (C) * 8 + (MC):                                                                                 \
    hipLaunchKernelGGL((k_decode_rows<FUSED, C, MC>), dim3(grid), dim3(kThreads), shm, s, abf, lda, ac,  \
                       as, ats, dyn, b, bs, bts, M, N, K, y, ldy);                                     \
    break;
#define FP4Q_ROWS_CASES(C) FP4Q_ROWS_CASE(C, 1) FP4Q_ROWS_CASE(C, 2) FP4Q_ROWS_CASE(C, 3) FP4Q_ROWS_CASE(C, 4)
  switch (ch * 8 + (int)M) {
    FP4Q_ROWS_CASES(1)
    FP4Q_ROWS_CASES(2)
    FP4Q_ROWS_CASES(3)
    FP4Q_ROWS_CASES(4)
    default: return hipErrorInvalidValue;
  }
#undef FP4Q_ROWS_CASES
#undef FP4Q_ROWS_CASE
  return hipGetLastError();
}

// ------------------------------------------------------- streamed form ----
//
// A workgroup owns a contiguous range of weight rows and walks it in 16-row
// groups.  Each group (16 rows x K: 40 KiB of codes + 5 KiB of scales at
// K = 5120) is pulled into LDS whole, by direct global->LDS loads issued back
// to back, so at any moment the chip reads a contiguous window of the weight
// rather than a thin K-slice of every row; two group buffers alternate.  The
// loads are placed in matrix-fragment order (load j, lane l: row l % 16,
// bytes 64 j + 16 (l / 16)), so every fragment read is one linear,
// conflict-free 16-byte LDS access.
//
// Sixteen wavefronts split K: wavefront w owns at most three 128-K steps, for
// which it holds the activation fragments already dequantized to fp16 in
// registers for the whole kernel, so per weight group it only dequantizes
// weight codes and runs the fp16 matrix core.  The sixteen partial tiles are
// summed in a fixed order through LDS by wavefronts 0-3, which also write the
// outputs; wavefronts 4-15 issue every direct load and wait on them with
// explicit vector-memory counts.  Scale bytes travel in 16-byte chunks: load j, lane l
// moves chunk (l / 16) + 4 j of row l % 16's scales.
constexpr int kStThreads = 1024;
constexpr int kStWaves = kStThreads / 64;
constexpr int kStMaxKT = 40;             // three group buffers + partial tiles within 160 KiB; K <= 5120
constexpr int kStKW = 3;                 // max 128-K steps per wavefront (ceil(40 / 16))
constexpr int kStNB = 3;                 // group buffers
// activation chunks per thread in the fused prologue: 8 x 5120 / 8 / 1024
// = 5 (M <= 8) and 16 x 5120 / 8 / 1024 = 10 (M <= 16)

// LDS: three group buffers of (KT + SJ) KiB, the third of which first holds
// the activation image (same layout, read once in the prologue), then the
// 16 wavefronts' partial tiles (16 x 4 x 64 floats).
struct StLayout {
  int KT, SJ;                            // 128-K steps; 1 KiB scale loads per group
  int buf, a_c, a_s, red, total;         // buf: bytes per group buffer
};
__host__ __device__ inline StLayout st_layout(int K) {
  StLayout L;
  L.KT = K / 128;
  L.SJ = (L.KT + 7) / 8;
  L.buf = (L.KT + L.SJ) * 1024;
  L.a_c = 2 * L.buf;
  L.a_s = 2 * L.buf + L.KT * 1024;
  L.red = 3 * L.buf;
  L.total = L.red + kStWaves * 4 * 64 * 4;
  return L;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p);
}
// one direct global->LDS load of 16 bytes per lane; lane l's bytes land at
// lds_base + 16 l.  No registers are written; completion is tracked by the
// explicit vector-memory waits below.
__device__ __forceinline__ void st_dma16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void wait_vmcnt(int n) {
#define FP4Q_VMW(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
  switch (n) {
    FP4Q_VMW(1) FP4Q_VMW(2) FP4Q_VMW(3) FP4Q_VMW(4) FP4Q_VMW(5) FP4Q_VMW(6) FP4Q_VMW(7) FP4Q_VMW(8)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
#undef FP4Q_VMW
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool FUSED, int ACTU>
__global__ __launch_bounds__(kStThreads) void k_decode_stream(
    const uint16_t* __restrict__ Abf, int64_t lda, const uint8_t* __restrict__ Ac,
    const uint8_t* __restrict__ As, float* Ats, int a_dynamic, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ Bts, int M, int N, int K, int rows_per_wg,
    float* __restrict__ Y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const StLayout L = st_layout(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int KT = L.KT, SJ = L.SJ, nsc = KT / 2;           // 16-byte scale chunks per row
  const uint32_t ldb = (uint32_t)K / 2, lds = (uint32_t)K / 16;
  const int row0 = blockIdx.x * rows_per_wg;
  const int row_end = min(N, row0 + rows_per_wg);
  const int G = (row_end - row0 + 15) / 16;
  const uint32_t sbase = lds_addr(smem);
  // scalars first: a later plain load would wait behind the direct loads
  const float bts = *Bts;
  const float ats_in = *Ats;

  // direct loads of one 16-row group into buffer s (wavefronts 4-15, which
  // issue no other vector-memory operation inside the loop, so their explicit
  // wait counts are exact; rows past the range re-read the last row, so every
  // lane of every load is active and the per-wavefront load count is the
  // same for every group)
  constexpr int kFirstDma = 4;
  const bool dma_wave = wave >= kFirstDma;
  const int dw = wave - kFirstDma, nd = kStWaves - kFirstDma;
  const int js0 = ((dw - KT) % nd + nd) % nd;             // first scale load of this wavefront
  auto issue_group = [&](int gi, int s) {
    const int r = min(row0 + gi * 16 + r16, row_end - 1);
    const uint32_t oc = (uint32_t)r * ldb + (uint32_t)g * 16u;
    const uint32_t os = (uint32_t)r * lds;
    const uint32_t bc = sbase + (uint32_t)(s * L.buf), bsc = bc + (uint32_t)(KT * 1024);
    for (int j = dw; j < KT; j += nd) st_dma16(B, oc + (uint32_t)j * 64u, bc + (uint32_t)j * 1024u);
    for (int j = js0; j < SJ; j += nd)
      st_dma16(Bs, os + (uint32_t)min(g + 4 * j, nsc - 1) * 16u, bsc + (uint32_t)j * 1024u);
  };
  int cnt = 0;
  if (dma_wave) {
    for (int j = dw; j < KT; j += nd) ++cnt;
    for (int j = js0; j < SJ; j += nd) ++cnt;
  }

  float ats;
  if constexpr (!FUSED) {
    if (dma_wave) {
      // activation codes and scales by the same direct loads (rows >= M
      // re-read row M - 1; their outputs are never stored)
      const int r = min(r16, M - 1);
      for (int j = dw; j < KT; j += nd)
        st_dma16(Ac, (uint32_t)r * ldb + (uint32_t)g * 16u + (uint32_t)j * 64u, sbase + (uint32_t)L.a_c + (uint32_t)j * 1024u);
      for (int j = js0; j < SJ; j += nd)
        st_dma16(As, (uint32_t)r * lds + (uint32_t)min(g + 4 * j, nsc - 1) * 16u, sbase + (uint32_t)L.a_s + (uint32_t)j * 1024u);
    }
    // every activation load is queued before any weight load: the vector
    // memory path returns in order, and the (cached) activation must not wait
    // behind the weight stream
    __builtin_amdgcn_s_barrier();
    if (dma_wave) {
      issue_group(0, 0);
      if (G > 1) issue_group(1, 1);
      wait_vmcnt(G > 1 ? 2 * cnt : cnt);                   // activation image complete
    }
    ats = ats_in;
  } else {
    // rows >= M of the image are zero
    for (int sl = tid; sl < KT * 64; sl += kStThreads)
      if ((sl & 15) >= M) *reinterpret_cast<uint4*>(smem + L.a_c + sl * 16) = uint4{0u, 0u, 0u, 0u};
    for (int sl = tid; sl < SJ * 64; sl += kStThreads)
      if ((sl & 15) >= M) *reinterpret_cast<uint4*>(smem + L.a_s + sl * 16) = uint4{0u, 0u, 0u, 0u};
    // paired scales: 2% faster at M = 4, 2% slower at M = 16 (the ten-chunk
    // form then needs 128 registers instead of 120)
    ats = quantize_act_block<kStThreads, ACTU, (ACTU <= 5)>(
        Abf, lda, M, K, ats_in, a_dynamic != 0, reinterpret_cast<float*>(smem + L.red),
        [&](int r, int c8, uint32_t p, uint32_t sb) {
          const int kt = c8 >> 4, k8 = c8 & 15;
          *reinterpret_cast<uint32_t*>(smem + L.a_c + kt * 1024 + (((k8 >> 2) << 4) + r) * 16 + (k8 & 3) * 4) = p;
          if (!(c8 & 1)) {
            const int b = c8 >> 1, ch = b >> 4;
            smem[L.a_s + (ch >> 2) * 1024 + (((ch & 3) << 4) + r) * 16 + (b & 15)] = (uint8_t)sb;
          }
        });
    if (a_dynamic && blockIdx.x == 0 && tid == 0) *Ats = ats;
    // the weight stream starts once the activation loads have returned (the
    // vector memory path returns in order, and a plain load waits for every
    // earlier load of its wavefront)
    if (dma_wave) {
      issue_group(0, 0);
      if (G > 1) issue_group(1, 1);
    }
  }
  lds_barrier();                                           // activation image complete

  // this wavefront's activation fragments, dequantized once
  const int kb = (wave * KT) / kStWaves, ke = ((wave + 1) * KT) / kStWaves;
  v8h ah[kStKW][4];
#pragma unroll
  for (int i = 0; i < kStKW; ++i) {
    const int kt = min(kb + i, KT - 1);
    const uint4 qa = *reinterpret_cast<const uint4*>(smem + L.a_c + kt * 1024 + lane * 16);
    const int c = kt >> 1;
    const int so = (c >> 2) * 1024 + (((c & 3) << 4) + r16) * 16 + ((kt & 1) << 3) + 2 * g;
    v2h sa0, sa1;
    e4m3x2_to_h2(*reinterpret_cast<const uint16_t*>(smem + L.a_s + so), sa0, sa1);
    ah[i][0] = dequant8(qa.x, sa0);
    ah[i][1] = dequant8(qa.y, sa0);
    ah[i][2] = dequant8(qa.z, sa1);
    ah[i][3] = dequant8(qa.w, sa1);
  }
  lds_barrier();                                           // the image's space becomes buffer 2
  if (dma_wave && G > 2) issue_group(2, 2);
  const float tsc = ats * bts;

  float* red = reinterpret_cast<float*>(smem + L.red);
  for (int gi = 0; gi < G; ++gi) {
    const int s = gi % kStNB;
    if (dma_wave) wait_vmcnt(min(G - 1 - gi, kStNB - 1) * cnt);   // groups after gi stay in flight
    lds_barrier();                                         // group gi in LDS

    // copy this wavefront's slice of the group to registers, so the buffer
    // can be refilled before the matrix work starts
    const uint8_t* bcode = smem + s * L.buf;
    const uint8_t* bscl = bcode + KT * 1024;
    uint4 qb[kStKW];
    uint32_t wsb[kStKW];
#pragma unroll
    for (int i = 0; i < kStKW; ++i) {
      const int kt = min(kb + i, KT - 1);
      qb[i] = *reinterpret_cast<const uint4*>(bcode + kt * 1024 + lane * 16);
      const int c = kt >> 1;
      wsb[i] = *reinterpret_cast<const uint16_t*>(bscl + (c >> 2) * 1024 + (((c & 3) << 4) + r16) * 16 +
                                                  ((kt & 1) << 3) + 2 * g);
    }
    lds_barrier();                                         // buffer s free
    if (dma_wave && gi + kStNB < G) issue_group(gi + kStNB, s);

    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kStKW; ++i) {
      if (kb + i < ke) {
        v2h sb0, sb1;
        e4m3x2_to_h2(wsb[i], sb0, sb1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i][0], dequant8(qb[i].x, sb0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i][1], dequant8(qb[i].y, sb0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i][2], dequant8(qb[i].z, sb1), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i][3], dequant8(qb[i].w, sb1), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    lds_barrier();                                         // partials in LDS
    if (tid < 256) {
      // thread t sums output (r, l) = (t / 64, t % 64) of the tile over the
      // 16 wavefronts in order; lane l of a tile holds column l % 16 and
      // row 4 (l / 16) + r
      const int r = tid >> 6;
      float v = red[r * 64 + lane];
#pragma unroll
      for (int w = 1; w < kStWaves; ++w) v = v + red[(w * 4 + r) * 64 + lane];
      const int nrow = min(16, row_end - (row0 + gi * 16));
      const int m = g * 4 + r;
      if (m < M && r16 < nrow) Y[m * ldy + row0 + gi * 16 + r16] = v * tsc;
    }
  }
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

bool skinny_supported(int64_t K) { return K <= SK_MAXK; }

bool stream_supported(int64_t N, int64_t K) {
  return K % 256 == 0 && K / 128 <= kStMaxKT && N * (K / 2) < (int64_t(1) << 32);
}

#ifndef FP4Q_DEC_ROWS_MAXM
#define FP4Q_DEC_ROWS_MAXM 1
#endif

// a_dynamic (fused form only): the activation tensor scale is computed from
// the activation's amax and written to a_ts.
hipError_t launch_gemm_nvfp4_skinny(const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                                    const uint8_t* a_scales, const float* a_ts, int a_dynamic,
                                    const uint8_t* b, const uint8_t* bs, const float* bts,
                                    int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                                    hipStream_t s) {
  float* ats = const_cast<float*>(a_ts);
  const bool fused = a_bf16 != nullptr;
  if (M > FP4Q_DEC_ROWS_MAXM && stream_supported(N, K)) {
    const StLayout L = st_layout((int)K);
    // spread the rows evenly over one workgroup per compute unit
    const int n_cu = device_cus();
    const int64_t groups = (N + 15) / 16;
    int64_t grid = groups < n_cu ? groups : n_cu;
    const int64_t rpw = (N + grid - 1) / grid;
    grid = (N + rpw - 1) / rpw;
    // allow the full 160 KiB of LDS, once per device (the attribute is set
    // with that device current)
    static std::atomic<int> attr_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
      const void* ks[3] = {reinterpret_cast<const void*>(&k_decode_stream<false, 1>),
                           reinterpret_cast<const void*>(&k_decode_stream<true, 5>),
                           reinterpret_cast<const void*>(&k_decode_stream<true, 10>)};
      for (const void* k : ks) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
      }
      attr_set[dev].store(1, std::memory_order_release);
    }
    auto launch = [&](auto kern) -> hipError_t {
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kStThreads), (size_t)L.total, s,
                         reinterpret_cast<const uint16_t*>(a_bf16), lda, a_codes, a_scales, ats,
                         fused ? a_dynamic : 0, b, bs, bts, (int)M, (int)N, (int)K, (int)rpw, y, ldy);
      return hipGetLastError();
    };
    if (!fused) return launch(&k_decode_stream<false, 1>);
    if (M <= 8) return launch(&k_decode_stream<true, 5>);
    return launch(&k_decode_stream<true, 10>);
  }
  if (M <= kRowsMaxM) {
    // at most four 16-byte chunks per lane: K / 32 <= 256 holds for K <= 7168
    const int ch = (int)((K / 32 + 63) / 64);
    const size_t shm_r = (size_t)M * K * 2;
    const unsigned grid = FP4Q_ROWS_GRID;
    if (fused)
      return launch_rows<true>(ch, grid, shm_r, s, reinterpret_cast<const uint16_t*>(a_bf16), lda, nullptr,
                               nullptr, ats, a_dynamic, b, bs, bts, M, N, K, y, ldy);
    return launch_rows<false>(ch, grid, shm_r, s, nullptr, (int64_t)0, a_codes, a_scales, ats, 0, b, bs, bts, M,
                              N, K, y, ldy);
  }
  if (fused && a_dynamic) {
    // this form reads the amax from the tensor-scale cell
    const hipError_t e = launch_amax_to_cell(a_bf16, 1, M, K, lda, ats, nullptr, 0, s);
    if (e != hipSuccess) return e;
  }
  // the activation tiles, and afterwards the K-half reduction buffer
  // (2 row groups x FRAGS x 4 x 64 floats), share the allocation
  const size_t shm_tiles = 16 * (K / 2 + 16) + 16 * (K / 16 + 4);
  const size_t shm_red = 2 * FRAGS * 4 * 64 * sizeof(float);
  const size_t shm = shm_tiles > shm_red ? shm_tiles : shm_red;
  if (fused)
    hipLaunchKernelGGL((k_decode<true>), dim3(cdiv(N, RPG)), dim3(kThreads), shm, s,
                       reinterpret_cast<const uint16_t*>(a_bf16), lda, nullptr, nullptr, ats, a_dynamic, b, bs,
                       bts, M, N, K, y, ldy);
  else
    hipLaunchKernelGGL((k_decode<false>), dim3(cdiv(N, RPG)), dim3(kThreads), shm, s, nullptr, (int64_t)0,
                       a_codes, a_scales, ats, 0, b, bs, bts, M, N, K, y, ldy);
  return hipGetLastError();
}

}  // namespace fp4q
