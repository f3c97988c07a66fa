// gemm_decode.hip -- decode-shaped NVFP4 W4A4 GEMM (M <= 16) for gfx950,
// with the activation quantization optionally fused into the prologue
// ("Why Gated DeltaNet Survives 4-Bit Quantization", limitations: decode was
// slowed by the separate small-batch NVFP4 activation-quantization kernel).
//
// The weight (N x K NVFP4, ~50 MB for 17408 x 5120) is read exactly once,
// so the kernel is an HBM stream with as little VALU work per weight byte as
// possible:
//  * a workgroup owns 64 weight rows; its four wavefronts are two row
//    groups (32 rows = two 16-row fragments each, so every dequantized
//    activation fragment feeds two matrix instructions) times two K halves;
//    the two K-half partials are summed in a fixed order through LDS, so the
//    fused and the pre-quantized entry points produce identical Y;
//  * the weight codes and E4M3 scales of the next PF stages (128 K elements
//    each) are in flight in registers while the current ones are consumed,
//    and the first group is issued before the activation prologue;
//  * the <= 16 activation rows live in LDS as NVFP4 codes + scales with
//    padded row strides (conflict-free fragment reads); the prologue copies
//    or quantizes (exactly the fp4q_quantize_nvfp4 recipe) only the M real
//    rows and zero-fills the rest;
//  * both operands are dequantized exactly to fp16 in registers
//    (code * s_b has at most 6 significant bits); E4M3 scales become fp16
//    with one v_cvt_scalef32_pk_f16_fp8 per two blocks; the fp16 matrix core
//    multiplies and the tensor scales are applied once at the end.

#include <hip/hip_runtime.h>
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
  const int KT = (int)(K / 128);
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
        if (kt < kt_end) {
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
        const uint4 qa = *reinterpret_cast<const uint4*>(lAc + r16 * lrow + (int64_t)kt * 64 + g * 16);
        const uint32_t wsa = *reinterpret_cast<const uint16_t*>(lAs + r16 * lsrow + (int64_t)kt * 8 + 2 * g);
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
#define FP4Q_ROWS_GRID 768   // three 4-wavefront workgroups per CU
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
  if constexpr (FUSED) {
    // quantize A[0:M) exactly as k_quant_nvfp4 does (one lane per 8 values,
    // lane pairs share a 16-block)
    const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(Ats));
    ats = (a_dynamic && (u & kAmaxFlag)) ? __uint_as_float(u & 0x7FFFFFFFu) / 1536.0f : __uint_as_float(u);
    const float six_st = 6.0f * ats;
    const int nch_pad = (nch + kThreads - 1) / kThreads * kThreads;   // all lanes join the DPP
    for (int c = tid; c < nch_pad; c += kThreads) {
      const bool in = c < nch;
      const int r = in ? c / cpr : 0, c8 = in ? c % cpr : 0;
      const uint4 q = *reinterpret_cast<const uint4*>(Abf + (int64_t)r * lda + c8 * 8);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
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
      if (in) put8(r, c8, (sc == 0.0f) ? 0u : p, sb);
    }
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
          const uint4 a0 = ap[2 * h], a1 = ap[2 * h + 1];
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

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

bool skinny_supported(int64_t K) { return K <= SK_MAXK; }

hipError_t launch_gemm_nvfp4_skinny(const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                                    const uint8_t* a_scales, const float* a_ts, int a_dynamic,
                                    const uint8_t* b, const uint8_t* bs, const float* bts,
                                    int64_t M, int64_t N, int64_t K, float* y, int64_t ldy,
                                    hipStream_t s) {
  if (M <= kRowsMaxM) {
    // at most four 16-byte chunks per lane: K / 32 <= 256 holds for K <= 7168
    const int ch = (int)((K / 32 + 63) / 64);
    const size_t shm_r = (size_t)M * K * 2;
    const unsigned grid = FP4Q_ROWS_GRID;
    if (a_bf16)
      return launch_rows<true>(ch, grid, shm_r, s, reinterpret_cast<const uint16_t*>(a_bf16), lda, nullptr,
                               nullptr, const_cast<float*>(a_ts), a_dynamic, b, bs, bts, M, N, K, y, ldy);
    return launch_rows<false>(ch, grid, shm_r, s, nullptr, (int64_t)0, a_codes, a_scales,
                              const_cast<float*>(a_ts), 0, b, bs, bts, M, N, K, y, ldy);
  }
  // the activation tiles, and afterwards the K-half reduction buffer
  // (2 row groups x FRAGS x 4 x 64 floats), share the allocation
  const size_t shm_tiles = 16 * (K / 2 + 16) + 16 * (K / 16 + 4);
  const size_t shm_red = 2 * FRAGS * 4 * 64 * sizeof(float);
  const size_t shm = shm_tiles > shm_red ? shm_tiles : shm_red;
  if (a_bf16)
    hipLaunchKernelGGL((k_decode<true>), dim3(cdiv(N, RPG)), dim3(kThreads), shm, s,
                       reinterpret_cast<const uint16_t*>(a_bf16), lda, nullptr, nullptr,
                       const_cast<float*>(a_ts), a_dynamic, b, bs, bts, M, N, K, y, ldy);
  else
    hipLaunchKernelGGL((k_decode<false>), dim3(cdiv(N, RPG)), dim3(kThreads), shm, s, nullptr, (int64_t)0,
                       a_codes, a_scales, const_cast<float*>(a_ts), 0, b, bs, bts, M, N, K, y, ldy);
  return hipGetLastError();
}

}  // namespace fp4q
