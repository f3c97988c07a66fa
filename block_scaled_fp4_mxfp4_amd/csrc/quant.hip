// quant.hip -- memory-bound quantization kernels of libfp4q for gfx950:
// tensor amax, NVFP4 and MXFP4 block quantization (with the fused balance
// scale and block-32 Hadamard rotation), the standalone rotation, the
// balance-scale calibration statistic and first-order Sigma-Delta
// re-quantization.
//
// Work mapping shared by the block kernels: one lane owns 8 consecutive
// elements of a row (one 16-byte load of bf16, two of fp32), so a wavefront
// reads 1 KiB (bf16) of contiguous memory per load instruction and writes
// its packed codes as one contiguous 256-byte store.  An NVFP4 16-block is
// spread over a lane pair, an MXFP4 32-block over a lane quad; the block
// maximum and the Hadamard butterflies between lanes use DPP quad
// permutations, so no LDS is touched.
//
// The arithmetic order follows the recipes stated in include/fp4q.h; each
// step is one binary32 operation (-ffp-contract=off, IEEE division).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.h"
#include "internal.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------- helpers ----

__device__ __forceinline__ float dpp_xor1(float v) {   // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {   // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float v[8]) {
  if constexpr (BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Eight values -> eight packed E2M1 codes (element 2i in the low nibble of
// byte i) with v_cvt_scalef32_pk_fp4_f32 at scale 1.0: round to nearest,
// ties to the even code, saturation at +-6, sign of zero kept -- the same
// function as e2m1_encode() (checked exhaustively near every decision point
// and on random finite inputs), two elements per instruction.
__device__ __forceinline__ uint32_t encode8_scaled(const float v[8], float rho) {
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0] * rho, v[1] * rho, 1.0f, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * rho, v[3] * rho, 1.0f, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * rho, v[5] * rho, 1.0f, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * rho, v[7] * rho, 1.0f, 3);
  return p;
}

// Tensor-scale cell encoding while a dynamic quantization is in flight:
// bit 31 set -> the low 31 bits are max|x| (non-negative binary32) and
// s_t = fl(A / 1536); bit 31 clear -> the cell already holds s_t.
constexpr uint32_t kAmaxFlag = 0x80000000u;

__device__ __forceinline__ float read_tensor_scale(const float* cell, int dynamic) {
  const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cell));
  if (dynamic && (u & kAmaxFlag)) return __uint_as_float(u & 0x7FFFFFFFu) / 1536.0f;
  return __uint_as_float(u);
}

// Element offset of chunk c (8 elements) in a [rows][ld] tensor whose rows
// hold cpr = cols/8 chunks.
template <bool CONTIG>
__device__ __forceinline__ int64_t chunk_offset(int64_t c, int64_t cpr, int64_t ld) {
  if constexpr (CONTIG) return c * 8;
  const int64_t r = c / cpr;
  return r * ld + (c - r * cpr) * 8;
}

// Chunk actually loaded for index c: past the end, the last chunk.  Loads
// stay unconditional -- a load under a branch makes the compiler wait for it
// before the next one is issued -- and what a clamped load brings in is
// never stored (nor can it change a maximum).
__device__ __forceinline__ int64_t clamp_chunk(int64_t c, int64_t n) { return c < n ? c : n - 1; }

// Row and column (in chunks) of chunk base + loc, rows of cpr chunks, with
// r0 = base / cpr and c0 = base % cpr computed once per workgroup (base is
// uniform): for rows of at least `span` chunks (loc < span) the column
// wraps at most once, so there is no per-thread division.
__device__ __forceinline__ void chunk_row_col(int64_t r0, int64_t c0, int loc, int span, int64_t cpr,
                                              int64_t& row, int64_t& col) {
  col = c0 + loc;
  row = r0;
  if (cpr >= span) {
    const bool wrap = col >= cpr;
    col = wrap ? col - cpr : col;
    row = wrap ? row + 1 : row;
  } else {
    row += col / cpr;
    col = col % cpr;
  }
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- amax ----

// Tensor maximum in two steps without atomics (many workgroups updating
// one address serialise in L2): each workgroup writes the bit pattern of
// its partial max|x| to partial[blockIdx.x]; a one-workgroup finalize
// kernel reduces the partials into the tensor-scale cell (amax encoding).
// With direct != 0 (single workgroup) the cell is written at once.
#ifndef FP4Q_AMAX_UNROLL
#define FP4Q_AMAX_UNROLL 8      // loads in flight per thread per iteration (measured best of 2, 4, 8)
#endif
constexpr int kAmaxUnroll = FP4Q_AMAX_UNROLL;
#ifndef FP4Q_AMAX_GRID
#define FP4Q_AMAX_GRID 512     // two workgroups per CU
#endif
constexpr int kAmaxMaxGrid = FP4Q_AMAX_GRID;

template <bool BF16, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_amax(const void* __restrict__ x, int64_t nchunks,
                                                   int64_t cpr, int64_t ld,
                                                   uint32_t* __restrict__ out, int direct) {
  // max|x| on the bit patterns: non-negative floats order like unsigned ints
  constexpr int W = BF16 ? 4 : 8;             // dwords per 8-element chunk
  uint32_t m = 0;
  us2 m2 = {0, 0};
  const int64_t stride = (int64_t)gridDim.x * kThreads * kAmaxUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kAmaxUnroll; base < nchunks; base += stride) {
    uint32_t raw[kAmaxUnroll][W];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {           // all loads first
      const int64_t c = clamp_chunk(base + u * kThreads + threadIdx.x, nchunks);
      const uint4* p = reinterpret_cast<const uint4*>(
          reinterpret_cast<const char*>(x) + chunk_offset<CONTIG>(c, cpr, ld) * (BF16 ? 2 : 4));
      const uint4 q = p[0];
      raw[u][0] = q.x; raw[u][1] = q.y; raw[u][2] = q.z; raw[u][3] = q.w;
      if constexpr (!BF16) {
        const uint4 q2 = p[1];
        raw[u][4] = q2.x; raw[u][5] = q2.y; raw[u][6] = q2.z; raw[u][7] = q2.w;
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
#pragma unroll
      for (int i = 0; i < W; ++i) {
        if constexpr (BF16) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(us2, raw[u][i] & 0x7FFF7FFFu));
        else m = max(m, raw[u][i] & 0x7FFFFFFFu);
      }
  }
  if constexpr (BF16) m = (uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16;
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
    if (direct) out[0] = kAmaxFlag | m;
    else out[blockIdx.x] = m;
  }
}

__global__ __launch_bounds__(kThreads) void k_amax_finalize(const uint32_t* __restrict__ partial, int n,
                                                            uint32_t* __restrict__ cell) {
  // every partial is loaded before any is used (n <= kAmaxMaxGrid = 2 x kThreads):
  // one memory latency, not one per element
  uint32_t q[kAmaxMaxGrid / kThreads];
#pragma unroll
  for (int j = 0; j < kAmaxMaxGrid / kThreads; ++j) {
    const int i = threadIdx.x + j * kThreads;
    q[j] = partial[i < n ? i : n - 1];
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kAmaxMaxGrid / kThreads; ++j) m = max(m, q[j]);     // non-negative floats
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
    // s_t itself (flag clear): the quantization kernel's threads then read
    // it instead of each dividing A by 1536
    *cell = __float_as_uint(__uint_as_float(m) / 1536.0f);
  }
}

// -------------------------------------------------------------- NVFP4 ----

#ifndef FP4Q_NV_UNROLL
#define FP4Q_NV_UNROLL 2        // 8-element chunks per thread (measured best of 1, 2, 4, 8)
#endif
constexpr int kNvUnroll = FP4Q_NV_UNROLL;

// Squared reconstruction error of a lane's 8 elements under packed codes p
// and total scale s, in the fixed order of the 4/6 rule:
// d_i = fl(x_i - fl(s * value(code_i))), e_i = fl(d_i * d_i),
// ((e0 + e1) + (e2 + e3)) + ((e4 + e5) + (e6 + e7)).
__device__ __forceinline__ float half_block_sq_error(const float v[8], uint32_t p, float s) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q0, q1;
    switch (i) {
      case 0: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0); q0 = q[0]; q1 = q[1]; break; }
      case 1: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1); q0 = q[0]; q1 = q[1]; break; }
      case 2: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2); q0 = q[0]; q1 = q[1]; break; }
      default: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3); q0 = q[0]; q1 = q[1]; break; }
    }
    const float d0 = v[2 * i] - s * q0, d1 = v[2 * i + 1] - s * q1;
    e[2 * i] = d0 * d0;
    e[2 * i + 1] = d1 * d1;
  }
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// FS: the 4/6 block scaling -- each block also tries the scale that maps its
// maximum to 4 and keeps it when the block's squared error is strictly
// smaller (both lanes of the pair add the two halves, so they agree).
template <bool BF16, bool CONTIG, bool FS>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(
    const void* __restrict__ x, int64_t nchunks, int64_t cpr, int64_t ld,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* ts, int dynamic) {
  const float st = read_tensor_scale(ts, dynamic);
  const float six_st = 6.0f * st;
  const float four_st = 4.0f * st;
  float v[kNvUnroll][8];
  int64_t cidx[kNvUnroll];
#pragma unroll
  for (int u = 0; u < kNvUnroll; ++u) {
    cidx[u] = ((int64_t)blockIdx.x * kNvUnroll + u) * kThreads + threadIdx.x;
    load8<BF16>(x, chunk_offset<CONTIG>(clamp_chunk(cidx[u], nchunks), cpr, ld), v[u]);
  }
  // Block maxima of every chunk (over the lane pair), then the block
  // scales: both lanes of a pair need the scales of both of their blocks,
  // so the even lane computes those of chunk u and the odd lane those of
  // chunk u + 1, and each passes its results to the other (the same
  // operations on the same operands, computed once per pair).
  static_assert(kNvUnroll % 2 == 0, "chunks are paired");
  const bool odd = threadIdx.x & 1;
  float a[kNvUnroll];
#pragma unroll
  for (int u = 0; u < kNvUnroll; ++u) {
    a[u] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[u] = fmaxf(a[u], __builtin_fabsf(v[u][i]));
    a[u] = fmaxf(a[u], dpp_xor1(a[u]));            // block max over the lane pair
  }
  uint32_t sbv[kNvUnroll], sb4v[FS ? kNvUnroll : 1];
  float sv[kNvUnroll], rv[kNvUnroll], s4v[FS ? kNvUnroll : 1], r4v[FS ? kNvUnroll : 1];
  auto scales_of = [&](float am, float div, uint32_t& sb, float& sc, float& rho) {
    sb = 0;
    if (am > 0.0f && st > 0.0f) sb = e4m3_ceil(am / div);
    sc = st * e4m3_decode(sb);
    rho = 1.0f / sc;
  };
  auto share = [&](uint32_t sb, float sc, float rho, uint32_t* sbo, float* so, float* ro, int u) {
    const uint32_t sbp = (uint32_t)__float_as_int(dpp_xor1(__int_as_float((int)sb)));
    const float sp = dpp_xor1(sc), rp = dpp_xor1(rho);
    sbo[u] = odd ? sbp : sb;
    so[u] = odd ? sp : sc;
    ro[u] = odd ? rp : rho;
    sbo[u + 1] = odd ? sb : sbp;
    so[u + 1] = odd ? sc : sp;
    ro[u + 1] = odd ? rho : rp;
  };
#pragma unroll
  for (int u = 0; u < kNvUnroll; u += 2) {
    const float am = odd ? a[u + 1] : a[u];
    uint32_t sb;
    float sc, rho;
    scales_of(am, six_st, sb, sc, rho);
    share(sb, sc, rho, sbv, sv, rv, u);
    if constexpr (FS) {
      scales_of(am, four_st, sb, sc, rho);
      share(sb, sc, rho, sb4v, s4v, r4v, u);
    }
  }
#pragma unroll
  for (int u = 0; u < kNvUnroll; ++u) {
    uint32_t sb = sbv[u];
    const float s = sv[u];
    uint32_t p = (s == 0.0f) ? 0u : encode8_scaled(v[u], rv[u]);
    if constexpr (FS) {
      const float s4 = s4v[u];
      const uint32_t p4 = (s4 == 0.0f) ? 0u : encode8_scaled(v[u], r4v[u]);
      const float h6 = half_block_sq_error(v[u], p, s), h4 = half_block_sq_error(v[u], p4, s4);
      const float e6 = h6 + dpp_xor1(h6), e4 = h4 + dpp_xor1(h4);
      if (e4 < e6) {
        sb = sb4v[u];
        p = p4;
      }
    }
    if (cidx[u] < nchunks) {
      codes[cidx[u]] = p;
      if (!(cidx[u] & 1)) scales[cidx[u] >> 1] = (uint8_t)sb;
    }
  }
  if (dynamic && blockIdx.x == 0 && threadIdx.x == 0) *ts = st;
}

// -------------------------------------------------------------- MXFP4 ----

// Per-lane part of the block-32 transform: z = x * t; stages h = 1, 2, 4
// inside the lane; h = 8 and h = 16 across the quad (lane bit 0 and bit 1);
// then times fl32(1/sqrt(32)).  The lower partner of every butterfly gets
// a + b, the upper one a - b, with a the lower element -- the same IEEE
// operations on the same operands as the sequential definition.
__device__ __forceinline__ void hadamard32_lane(float z[8], int qlane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = z[i], b = z[i + h];
      z[i] = a + b;
      z[i + h] = a - b;
    }
  }
  const bool up1 = qlane & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dpp_xor1(z[i]);
    z[i] = up1 ? (o - z[i]) : (z[i] + o);
  }
  const bool up2 = qlane & 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dpp_xor2(z[i]);
    z[i] = up2 ? (o - z[i]) : (z[i] + o);
  }
  const float c = 0.17677669529663687f;   // fl32(1/sqrt(32)) = 0x3E3504F3
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = z[i] * c;
}

__device__ __forceinline__ void apply_chan_scale(float z[8], const float* __restrict__ t,
                                                 int64_t col) {
  const float4* p = reinterpret_cast<const float4*>(t + col);
  const float4 a = p[0], b = p[1];
  z[0] = z[0] * a.x; z[1] = z[1] * a.y; z[2] = z[2] * a.z; z[3] = z[3] * a.w;
  z[4] = z[4] * b.x; z[5] = z[5] * b.y; z[6] = z[6] * b.z; z[7] = z[7] * b.w;
}

#ifndef FP4Q_MX_UNROLL
#define FP4Q_MX_UNROLL 2
#endif
constexpr int kMxUnroll = FP4Q_MX_UNROLL;

template <bool BF16, bool CONTIG, bool SCALE, bool HAD>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(
    const void* __restrict__ x, int64_t nchunks, int64_t cpr, int64_t ld,
    const float* __restrict__ t, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  float v[kMxUnroll][8], ts[SCALE ? kMxUnroll : 1][8];
  int64_t cidx[kMxUnroll];
  const int64_t base = (int64_t)blockIdx.x * kMxUnroll * kThreads;
  const int64_t r0 = SCALE ? base / cpr : 0, c0 = SCALE ? base - r0 * cpr : 0;   // uniform
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {              // all loads first
    cidx[u] = base + u * kThreads + threadIdx.x;
    const int64_t cl = clamp_chunk(cidx[u], nchunks);
    load8<BF16>(x, chunk_offset<CONTIG>(cl, cpr, ld), v[u]);
    if constexpr (SCALE) {
      // the channel scales of chunk cidx's column (past the end: some
      // in-range column; that chunk is not stored)
      int64_t row, col;
      chunk_row_col(r0, c0, u * kThreads + (int)threadIdx.x, kMxUnroll * kThreads, cpr, row, col);
      load8<false>(t, col * 8, ts[u]);
    }
  }
  const int qlane = threadIdx.x & 3;
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {
    if constexpr (SCALE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = v[u][i] * ts[u][i];
    }
    if constexpr (HAD) hadamard32_lane(v[u], qlane);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[u][i]));
    a = fmaxf(a, dpp_xor1(a));
    a = fmaxf(a, dpp_xor2(a));
    const bool zero = !(a > 0.0f);
    const int32_t e = zero ? -127 : mx_block_exponent(a);
    const float inv = pow2_neg(e);
    const uint32_t p = zero ? 0u : encode8_scaled(v[u], inv);
    if (cidx[u] < nchunks) {
      codes[cidx[u]] = p;
      if (qlane == 0) scales[cidx[u] >> 2] = (uint8_t)(e + 127);
    }
  }
}

template <bool BF16, bool CONTIG, bool SCALE>
__global__ __launch_bounds__(kThreads) void k_hadamard32(
    const void* __restrict__ x, int64_t nchunks, int64_t cpr, int64_t ld,
    const float* __restrict__ t, float* __restrict__ y, int64_t ldy) {
  const int64_t base = (int64_t)blockIdx.x * kThreads;
  const int64_t c = base + threadIdx.x;
  const int64_t cl = clamp_chunk(c, nchunks);
  const int64_t r0 = base / cpr, c0 = base - r0 * cpr;                         // uniform
  int64_t row, col;                                  // of chunk c
  chunk_row_col(r0, c0, (int)threadIdx.x, kThreads, cpr, row, col);
  float v[8];
  load8<BF16>(x, chunk_offset<CONTIG>(cl, cpr, ld), v);
  if constexpr (SCALE) apply_chan_scale(v, t, col * 8);   // past the end: an in-range column, not stored
  hadamard32_lane(v, threadIdx.x & 3);
  if (c < nchunks) {
    float4* p = reinterpret_cast<float4*>(y + row * ldy + col * 8);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ------------------------------------------------------ balance scale ----

// One workgroup per 64 columns: 4 row-lanes x 64 column-lanes; fp64 column
// sums, two passes for the standard deviation (mean first).
template <bool BF16>
__device__ __forceinline__ double load1(const void* p, int64_t off) {
  if constexpr (BF16) return (double)bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[off]);
  return (double)reinterpret_cast<const float*>(p)[off];
}

template <bool WBF16, bool XBF16>
__global__ __launch_bounds__(kThreads) void k_balance(const void* __restrict__ w, int64_t N,
                                                      int64_t K, int64_t ldw,
                                                      const void* __restrict__ x, int64_t M,
                                                      int64_t ldx, double alpha,
                                                      float* __restrict__ t_out,
                                                      float* __restrict__ u_out) {
  __shared__ double red[4][64];
  const int cl = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 64 + cl;
  const bool ok = col < K;
  // pass 1: column mean of W
  double s = 0.0;
  if (ok)
    for (int64_t r = rl; r < N; r += 4) s += load1<WBF16>(w, r * ldw + col);
  red[rl][cl] = s;
  __syncthreads();
  const double mean = (red[0][cl] + red[1][cl] + red[2][cl] + red[3][cl]) / (double)N;
  __syncthreads();
  // pass 2: sum of squared deviations
  s = 0.0;
  if (ok)
    for (int64_t r = rl; r < N; r += 4) {
      const double d = load1<WBF16>(w, r * ldw + col) - mean;
      s += d * d;
    }
  red[rl][cl] = s;
  __syncthreads();
  const double var = (red[0][cl] + red[1][cl] + red[2][cl] + red[3][cl]) / (double)N;
  __syncthreads();
  // activation column mean square
  s = 0.0;
  if (ok)
    for (int64_t r = rl; r < M; r += 4) {
      const double v = load1<XBF16>(x, r * ldx + col);
      s += v * v;
    }
  red[rl][cl] = s;
  __syncthreads();
  if (rl == 0 && ok) {
    const double ms = (red[0][cl] + red[1][cl] + red[2][cl] + red[3][cl]) / (double)M;
    const double sigma = fmax(sqrt(var), 1e-12);
    const double rms = fmax(sqrt(ms), 1e-12);
    double tt = pow(sigma, alpha) / pow(rms, 1.0 - alpha);
    tt = fmin(fmax(tt, 0x1p-16), 0x1p16);
    t_out[col] = (float)tt;
    u_out[col] = (float)(1.0 / tt);
  }
}

// -------------------------------------------------------- Sigma-Delta ----

constexpr int kSdMaxSeg = 16;

struct SdArgs {
  const float* w[kSdMaxSeg];
  const uint8_t* scales[kSdMaxSeg];
  const float* ts[kSdMaxSeg];
  float* res[kSdMaxSeg];
  uint8_t* codes[kSdMaxSeg];
  int64_t nchunks[kSdMaxSeg];
  int32_t wg_start[kSdMaxSeg + 1];
  int32_t nseg;
};

#ifndef FP4Q_SD_UNROLL
#define FP4Q_SD_UNROLL 2        // chunks per thread
#endif
constexpr int kSdUnroll = FP4Q_SD_UNROLL;

// SCHED: the reverse-order tail schedule -- the chain starts from r = 0 on
// chip (no residue buffer), runs `steps` = K steps, writes step k (0-based)
// to bank n_rtn + K - 1 - k and, at k = 0, the same codes (the nearest
// codes) to banks 0 .. n_rtn - 1.
template <bool SCHED>
__global__ __launch_bounds__(kThreads) void k_sigma_delta(const SdArgs args, int steps,
                                                          int64_t bank_stride, int n_rtn) {
  int seg = 0;
  while (seg + 1 < args.nseg && (int)blockIdx.x >= args.wg_start[seg + 1]) ++seg;
  const int64_t wg = (int64_t)blockIdx.x - args.wg_start[seg];
  const int64_t n = args.nchunks[seg];
  const float st = *args.ts[seg];
  const float* __restrict__ w = args.w[seg];
  float* __restrict__ res = args.res[seg];
  float x[kSdUnroll][8], r[kSdUnroll][8];
  int64_t cidx[kSdUnroll];
  uint32_t sb_raw[kSdUnroll];
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u) {              // all loads first
    cidx[u] = (wg * kSdUnroll + u) * kThreads + threadIdx.x;
    const int64_t cl = clamp_chunk(cidx[u], n);
    load8<false>(w, cl * 8, x[u]);
    if (SCHED) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r[u][i] = 0.0f;
    } else {
      load8<false>(res, cl * 8, r[u]);
    }
    sb_raw[u] = args.scales[seg][cl >> 1];
  }
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u) {
    const bool in = cidx[u] < n;
    const uint32_t sb = in ? sb_raw[u] : 0u;
    const float s = st * e4m3_decode(sb);
    const float rho = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float xi = in ? x[u][i] * rho : 0.0f;
      if (!(s != 0.0f)) xi = 0.0f;
      xi = fminf(fmaxf(xi, -6.0f), 6.0f);
      x[u][i] = xi;
      if (!in) r[u][i] = 0.0f;
    }
  }
  uint8_t* codes = args.codes[seg];
  for (int k = 0; k < steps; ++k) {
#pragma unroll
    for (int u = 0; u < kSdUnroll; ++u) {
      // per element pair: v = x + r; code = nearest E2M1 (hardware convert,
      // same function as e2m1_encode); r = v - value(code), exact.
      uint32_t pk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v0 = x[u][2 * i] + r[u][2 * i], v1 = x[u][2 * i + 1] + r[u][2 * i + 1];
        switch (i) {
          case 0: pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, v0, v1, 1.0f, 0); break;
          case 1: pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, v0, v1, 1.0f, 1); break;
          case 2: pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, v0, v1, 1.0f, 2); break;
          default: pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, v0, v1, 1.0f, 3); break;
        }
        float q0, q1;
        switch (i) {
          case 0: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 0); q0 = q[0]; q1 = q[1]; break; }
          case 1: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 1); q0 = q[0]; q1 = q[1]; break; }
          case 2: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 2); q0 = q[0]; q1 = q[1]; break; }
          default: { auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk, 1.0f, 3); q0 = q[0]; q1 = q[1]; break; }
        }
        r[u][2 * i] = v0 - q0;
        r[u][2 * i + 1] = v1 - q1;
      }
      if (cidx[u] < n) {
        const int64_t bank = SCHED ? (int64_t)(n_rtn + steps - 1 - k) : (int64_t)k;
        reinterpret_cast<uint32_t*>(codes + bank * bank_stride)[cidx[u]] = pk;
        if (SCHED && k == 0)
          for (int b = 0; b < n_rtn; ++b) reinterpret_cast<uint32_t*>(codes + (int64_t)b * bank_stride)[cidx[u]] = pk;
      }
    }
  }
  if (SCHED) return;
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u) {
    if (cidx[u] < n) {
      float4* p = reinterpret_cast<float4*>(res + cidx[u] * 8);
      p[0] = make_float4(r[u][0], r[u][1], r[u][2], r[u][3]);
      p[1] = make_float4(r[u][4], r[u][5], r[u][6], r[u][7]);
    }
  }
}

// ------------------------------------------------- stochastic rounding ----
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of
// (c0..c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// with the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;   // one 32x32->64 each
    // three-input exclusive or in one instruction (truth table 0x96)
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

// Stochastic rounding of x in [-6, 6] to an E2M1 code with one random word
// (sr_prepare once per element, sr_pick once per access):
// lo = the largest E2M1 value <= x, hi = the next one; u = (word >> 8) 2^-24;
// hi exactly when lo + u (hi - lo) < x, so P(hi) = (x - lo) / (hi - lo) up to
// 2^-24.  Evaluated exactly in integers: with s = 2^24 / (hi - lo) (a power
// of two), the test is lo s + U < x s for the integer U = word >> 8, and
// for an integer left side that is lo s + U < ceil(x s); lo s and x s are
// exact binary32 products below 2^28 in magnitude.  Values on the grid are
// kept; a zero value keeps the sign bit of x.
// Bracket of x: lo, the largest E2M1 value <= x, as a code, and whether a
// next value hi exists; hi's code is lo's plus one (x >= 0) or minus one
// (x < 0: magnitudes fall towards zero).
__device__ __forceinline__ uint32_t bracket_lo(float x, bool& has_hi) {
  const float a = __builtin_fabsf(x);
  const uint32_t fl = (a >= 0.5f) + (a >= 1.0f) + (a >= 1.5f) + (a >= 2.0f) + (a >= 3.0f) + (a >= 4.0f) + (a >= 6.0f);
  if (__float_as_uint(x) >> 31) {
    const uint32_t ce = fl + (e2m1_decode(fl) < a ? 1u : 0u);     // smallest magnitude >= a
    has_hi = ce > 0u;
    return ce | 8u;
  }
  has_hi = fl < 7u;
  return fl;
}
__device__ __forceinline__ uint32_t bracket_hi(uint32_t lo_c) { return (lo_c & 8u) ? lo_c - 1u : lo_c + 1u; }

// Per-element state of the stochastic rounding: (C - L) << 4 | code(lo),
// C - L in [0, 2^24] (0 when x has no upper neighbour).
__device__ __forceinline__ uint32_t sr_prepare(float x) {
  bool has_hi;
  const uint32_t lo_c = bracket_lo(x, has_hi);
  if (!has_hi) return lo_c;
  const float lo = e2m1_decode(lo_c);
  // 2^24 / (hi - lo) from the exponent field of hi - lo (0.5, 1 or 2)
  const float sc = __uint_as_float((278u - (__float_as_uint(e2m1_decode(bracket_hi(lo_c)) - lo) >> 23)) << 23);
  const int32_t diff = (int32_t)__builtin_ceilf(x * sc) - (int32_t)(lo * sc);
  return ((uint32_t)diff << 4) | lo_c;
}
__device__ __forceinline__ uint32_t sr_pick(uint32_t state, uint32_t word) {
  const uint32_t lo_c = state & 15u;
  return (word >> 8) < (state >> 4) ? bracket_hi(lo_c) : lo_c;
}

// A binary32 y in [0, 1] as m 2^-sh with its 24-bit significand m; sh is
// clamped to 63, which changes no floor or ceiling below: k m < 2^48.
__device__ __forceinline__ void split_unit(float y, uint32_t& m, uint32_t& sh) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t e = b >> 23;                                      // y >= 0
  m = e ? ((b & 0x7FFFFFu) | 0x800000u) : (b & 0x7FFFFFu);
  const uint32_t s = e ? 150u - e : 149u;
  sh = s < 63u ? s : 63u;
}

// Access k >= 1 of the stateless two-point chain (F4b; two_point_prepare
// and two_point_start once per element, two_point_next once per access):
// lo, hi the E2M1
// neighbours of x, p = (x - lo) / (hi - lo); hi exactly when
// floor(k p) - floor((k - 1) p) = 1.  Exact in integers for k < 2^24: x - lo
// is exact in binary32 (lo = 0, or Sterbenz: lo <= x <= 2 lo in magnitude)
// and hi - lo is a power of two, so p = m 2^-sh exactly and
// floor(k p) = (k m) >> sh; on [-0.5, 0), k p = k - k v with v = 2 |x|, so
// floor(k p) = k - ceil(k v), ceil(k v) = (k m + 2^sh - 1) >> sh.
// Per-element state of the two-point chain: w0 = m | code(lo) << 24 |
// neg0 << 28, w1 = sh (m = 0 when x has no upper neighbour or lies on the
// grid, which makes every access take lo).
__device__ __forceinline__ void two_point_prepare(float x, uint32_t& w0, uint32_t& w1) {
  bool has_hi;
  const uint32_t lo_c = bracket_lo(x, has_hi);
  if (!has_hi) { w0 = lo_c << 24; w1 = 0u; return; }
  const uint32_t hi_c = bracket_hi(lo_c);
  const bool neg0 = hi_c == 8u;                       // x in [-0.5, 0)
  const float lo = e2m1_decode(lo_c);
  // 1 / (hi - lo) from the exponent field of hi - lo (0.5, 1 or 2): exact
  const float inv = __uint_as_float((254u - (__float_as_uint(e2m1_decode(hi_c) - lo) >> 23)) << 23);
  const float y = neg0 ? 2.0f * __builtin_fabsf(x) : (x - lo) * inv;   // v or p, exact
  uint32_t m, sh;
  split_unit(y, m, sh);
  w0 = m | (lo_c << 24) | (neg0 ? 1u << 28 : 0u);
  w1 = sh;
}
// The accesses run in order, so the difference of floors is a carry: with
// T = 2^sh, bias = T - 1 on [-0.5, 0) (ceiling) else 0, and
// r = ((k - 1) m + bias) mod T, floor((k m + bias) / T) -
// floor(((k - 1) m + bias) / T) = [r + m >= T] (r < T and m <= T).
// two_point_start gives r before access k0 + 1; two_point_next takes one
// access: it adds m, reduces by the carry and picks the code.
__device__ __forceinline__ uint64_t two_point_start(uint32_t w0, uint32_t w1, uint32_t k0) {
  const uint32_t m = w0 & 0xFFFFFFu;
  const bool neg0 = (w0 >> 28) & 1u;
  const uint64_t t = uint64_t(1) << w1;
  return ((uint64_t)k0 * m + (neg0 ? t - 1u : 0u)) & (t - 1u);
}
__device__ __forceinline__ uint32_t two_point_next(uint32_t w0, uint32_t w1, uint64_t& r) {
  const uint32_t m = w0 & 0xFFFFFFu, lo_c = (w0 >> 24) & 15u;
  const bool neg0 = (w0 >> 28) & 1u;
  const uint64_t t = uint64_t(1) << w1;
  r += m;
  const bool carry = r >= t;
  r = carry ? r - t : r;
  return carry != neg0 ? bracket_hi(lo_c) : lo_c;
}

// `steps` accesses of stochastic rounding at the fixed NVFP4 scale of each
// segment (x = clamp(w / s, -6, 6), as the Sigma-Delta chain), access k
// written to bank k.  Element e (row-major within its segment) draws output
// word e mod 4 of Philox4x32-10 at counter (g lo, g hi, step0 + k, segment
// index) with g = e / 4, key (k0, k1).
// TWO_POINT: the two-point chain instead, bank k holding access
// step0 + k + 1 (no random words).
template <bool TWO_POINT>
__global__ __launch_bounds__(kThreads) void k_stochastic_round(const SdArgs args, int steps, int64_t bank_stride,
                                                               uint32_t k0, uint32_t k1, uint32_t step0,
                                                               int seg_base) {
  int seg = 0;
  while (seg + 1 < args.nseg && (int)blockIdx.x >= args.wg_start[seg + 1]) ++seg;
  const int64_t wg = (int64_t)blockIdx.x - args.wg_start[seg];
  const int64_t n = args.nchunks[seg];
  const float st = *args.ts[seg];
  float x[kSdUnroll][8];
  int64_t cidx[kSdUnroll];
  uint32_t sb_raw[kSdUnroll];
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u) {
    cidx[u] = (wg * kSdUnroll + u) * kThreads + threadIdx.x;
    const int64_t cl = clamp_chunk(cidx[u], n);
    load8<false>(args.w[seg], cl * 8, x[u]);
    sb_raw[u] = args.scales[seg][cl >> 1];
  }
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u) {
    const bool in = cidx[u] < n;
    const float s = st * e4m3_decode(in ? sb_raw[u] : 0u);
    const float rho = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float xi = in ? x[u][i] * rho : 0.0f;
      if (!(s != 0.0f)) xi = 0.0f;
      x[u][i] = fminf(fmaxf(xi, -6.0f), 6.0f);
    }
  }
  uint8_t* codes = args.codes[seg];
  const uint32_t sid = (uint32_t)(seg_base + seg);
  // per-element state, computed once for all accesses
  uint32_t w0[kSdUnroll][8], w1[kSdUnroll][8];
#pragma unroll
  for (int u = 0; u < kSdUnroll; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (TWO_POINT) two_point_prepare(x[u][i], w0[u][i], w1[u][i]);
      else w0[u][i] = sr_prepare(x[u][i]);
    }
  uint64_t tp_r[TWO_POINT ? kSdUnroll : 1][8];
  if constexpr (TWO_POINT) {
#pragma unroll
    for (int u = 0; u < kSdUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) tp_r[u][i] = two_point_start(w0[u][i], w1[u][i], step0);
  }
  for (int k = 0; k < steps; ++k) {
#pragma unroll
    for (int u = 0; u < kSdUnroll; ++u) {
      if (cidx[u] >= n) continue;
      uint32_t pk = 0;
      if constexpr (TWO_POINT) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pk |= two_point_next(w0[u][i], w1[u][i], tp_r[u][i]) << (4 * i);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {                    // two Philox groups of four elements
          const uint64_t g = (uint64_t)cidx[u] * 2 + h;
          const uint4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), step0 + (uint32_t)k, sid, k0, k1);
          pk |= sr_pick(w0[u][4 * h + 0], r.x) << (16 * h);
          pk |= sr_pick(w0[u][4 * h + 1], r.y) << (16 * h + 4);
          pk |= sr_pick(w0[u][4 * h + 2], r.z) << (16 * h + 8);
          pk |= sr_pick(w0[u][4 * h + 3], r.w) << (16 * h + 12);
        }
      }
      reinterpret_cast<uint32_t*>(codes + (int64_t)k * bank_stride)[cidx[u]] = pk;
    }
  }
}

// ------------------------------------------ fused-member harmonization ----
// One shared tensor scale for the members of a fused NVFP4 GEMM: s_t is the
// largest member scale; member i's block scales become the E4M3 value
// nearest to fl(s_b * fl(s_t,i / s_t)), codes untouched.  Bytes that are
// not a non-negative finite E4M3 value are left as they are.  A member with
// ratio 1 is left as it is (the rewrite is the identity there).
//
// Work split: a member's bytes are a 16-byte aligned body of 16-byte chunks
// plus at most 30 edge bytes (before the first aligned address and after
// the last whole chunk).  Item c < nchunk is body chunk c; item nchunk is
// the edge, done byte by byte by one thread.

constexpr int kHzMaxMem = 16;

struct HzArgs {
  uint8_t* scales[kHzMaxMem];
  const float* ts[kHzMaxMem];
  int64_t nbytes[kHzMaxMem];
  int32_t head[kHzMaxMem];           // bytes before the first 16-byte aligned address
  int32_t wg_start[kHzMaxMem + 1];
  int32_t n;
};

#ifndef FP4Q_HZ_UNROLL
#define FP4Q_HZ_UNROLL 2        // 16-byte chunks per thread
#endif
constexpr int kHzUnroll = FP4Q_HZ_UNROLL;

__device__ __forceinline__ uint32_t harmonize_byte(uint32_t b, float r) {
  return b <= 0x7Eu ? e4m3_round_nearest(e4m3_decode(b) * r) : b;
}

__device__ __forceinline__ uint32_t harmonize_word(uint32_t w, float r) {
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) o |= harmonize_byte((w >> (8 * j)) & 0xFFu, r) << (8 * j);
  return o;
}

__global__ __launch_bounds__(kThreads) void k_harmonize(const HzArgs a) {
  int m = 0;
  while (m + 1 < a.n && (int)blockIdx.x >= a.wg_start[m + 1]) ++m;
  float st = 0.0f;
  for (int i = 0; i < a.n; ++i) st = fmaxf(st, *a.ts[i]);
  const float r = st > 0.0f ? *a.ts[m] / st : 1.0f;
  if (r == 1.0f) return;                               // uniform over the workgroup
  uint8_t* __restrict__ p = a.scales[m];
  const int64_t nb = a.nbytes[m], head = a.head[m];
  const int64_t nchunk = (nb - head) >> 4;
  const int64_t wg = (int64_t)blockIdx.x - a.wg_start[m];
  auto* body = reinterpret_cast<uint4*>(p + head);
  int64_t c[kHzUnroll];
  bool edge = false;
#pragma unroll
  for (int u = 0; u < kHzUnroll; ++u) {
    c[u] = (wg * kHzUnroll + u) * kThreads + threadIdx.x;
    edge |= c[u] == nchunk;
  }
  if (nchunk > 0) {                                     // uniform
    uint4 v[kHzUnroll];
#pragma unroll
    for (int u = 0; u < kHzUnroll; ++u) v[u] = body[clamp_chunk(c[u], nchunk)];
#pragma unroll
    for (int u = 0; u < kHzUnroll; ++u) {
      if (c[u] < nchunk) {
        uint4 o;
        o.x = harmonize_word(v[u].x, r);
        o.y = harmonize_word(v[u].y, r);
        o.z = harmonize_word(v[u].z, r);
        o.w = harmonize_word(v[u].w, r);
        body[c[u]] = o;
      }
    }
  }
  if (edge) {                                           // one thread of the member
    for (int64_t i = 0; i < head; ++i) p[i] = (uint8_t)harmonize_byte(p[i], r);
    for (int64_t i = head + nchunk * 16; i < nb; ++i) p[i] = (uint8_t)harmonize_byte(p[i], r);
  }
}

// After every member is rewritten: all member cells and the shared cell
// take the shared scale (one thread, so aliased cells are harmless).
__global__ void k_harmonize_cells(const HzArgs a, float* shared) {
  if (threadIdx.x != 0) return;
  float st = 0.0f;
  for (int i = 0; i < a.n; ++i) st = fmaxf(st, *a.ts[i]);
  for (int i = 0; i < a.n; ++i) *const_cast<float*>(a.ts[i]) = st;
  *shared = st;
}

inline unsigned grid_for(int64_t items, int64_t per_block) {
  return (unsigned)((items + per_block - 1) / per_block);
}

}  // namespace

// ------------------------------------------------------------ launchers ----

hipError_t launch_amax_to_cell(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                               float* cell, uint8_t* scratch, int64_t scratch_bytes, hipStream_t s) {
  const int64_t cpr = cols / 8, n = rows * cpr;
  const bool contig = (ldx == cols);
  int64_t g = grid_for(n, (int64_t)kThreads * kAmaxUnroll * 2);    // ~2 iterations per thread
  if (g > kAmaxMaxGrid) g = kAmaxMaxGrid;
  if (g > scratch_bytes / 4) g = scratch_bytes / 4;
  if (g < 1) g = 1;
  const int direct = (g == 1);
  uint32_t* out = direct ? reinterpret_cast<uint32_t*>(cell) : reinterpret_cast<uint32_t*>(scratch);
  if (bf16) {
    if (contig) hipLaunchKernelGGL((k_amax<true, true>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ldx, out, direct);
    else hipLaunchKernelGGL((k_amax<true, false>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ldx, out, direct);
  } else {
    if (contig) hipLaunchKernelGGL((k_amax<false, true>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ldx, out, direct);
    else hipLaunchKernelGGL((k_amax<false, false>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ldx, out, direct);
  }
  if (!direct)
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(scratch),
                       (int)g, reinterpret_cast<uint32_t*>(cell));
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* ts, int ts_is_input,
                              int four_six, hipStream_t s) {
  const int dynamic = !ts_is_input;
  if (dynamic) {
    // the block-scale output doubles as scratch for the partial maxima; the
    // quantization pass overwrites it afterwards (stream order)
    hipError_t e = launch_amax_to_cell(x, bf16, rows, cols, ldx, ts, scales, rows * (cols / 16), s);
    if (e != hipSuccess) return e;
  }
  const int64_t cpr = cols / 8, n = rows * cpr;
  const bool contig = (ldx == cols);
  const unsigned g = grid_for(n, (int64_t)kThreads * kNvUnroll);
  auto* c32 = reinterpret_cast<uint32_t*>(codes);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), 0, s, x, n, cpr, ldx, c32, scales, ts, dynamic);
  };
  if (four_six) {
    if (bf16) contig ? go(k_quant_nvfp4<true, true, true>) : go(k_quant_nvfp4<true, false, true>);
    else contig ? go(k_quant_nvfp4<false, true, true>) : go(k_quant_nvfp4<false, false, true>);
  } else {
    if (bf16) contig ? go(k_quant_nvfp4<true, true, false>) : go(k_quant_nvfp4<true, false, false>);
    else contig ? go(k_quant_nvfp4<false, true, false>) : go(k_quant_nvfp4<false, false, false>);
  }
  return hipGetLastError();
}

namespace {
template <bool BF16, bool CONTIG>
void launch_mx_variant(bool scale, bool had, unsigned g, hipStream_t s, const void* x, int64_t n,
                       int64_t cpr, int64_t ld, const float* t, uint32_t* c, uint8_t* sc) {
  if (scale && had) hipLaunchKernelGGL((k_quant_mxfp4<BF16, CONTIG, true, true>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, c, sc);
  else if (scale) hipLaunchKernelGGL((k_quant_mxfp4<BF16, CONTIG, true, false>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, c, sc);
  else if (had) hipLaunchKernelGGL((k_quant_mxfp4<BF16, CONTIG, false, true>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, c, sc);
  else hipLaunchKernelGGL((k_quant_mxfp4<BF16, CONTIG, false, false>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, c, sc);
}
template <bool BF16, bool CONTIG>
void launch_had_variant(bool scale, unsigned g, hipStream_t s, const void* x, int64_t n,
                        int64_t cpr, int64_t ld, const float* t, float* y, int64_t ldy) {
  if (scale) hipLaunchKernelGGL((k_hadamard32<BF16, CONTIG, true>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, y, ldy);
  else hipLaunchKernelGGL((k_hadamard32<BF16, CONTIG, false>), dim3(g), dim3(kThreads), 0, s, x, n, cpr, ld, t, y, ldy);
}
}  // namespace

hipError_t launch_quant_mxfp4(const void* x, int bf16, int64_t rows, int64_t cols, int64_t ldx,
                              const float* chan_scale, int hadamard, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t cpr = cols / 8, n = rows * cpr;
  const bool contig = (ldx == cols);
  const unsigned g = grid_for(n, (int64_t)kThreads * kMxUnroll);
  auto* c32 = reinterpret_cast<uint32_t*>(codes);
  const bool sc = chan_scale != nullptr, had = hadamard != 0;
  if (bf16) {
    if (contig) launch_mx_variant<true, true>(sc, had, g, s, x, n, cpr, ldx, chan_scale, c32, scales);
    else launch_mx_variant<true, false>(sc, had, g, s, x, n, cpr, ldx, chan_scale, c32, scales);
  } else {
    if (contig) launch_mx_variant<false, true>(sc, had, g, s, x, n, cpr, ldx, chan_scale, c32, scales);
    else launch_mx_variant<false, false>(sc, had, g, s, x, n, cpr, ldx, chan_scale, c32, scales);
  }
  return hipGetLastError();
}

hipError_t launch_hadamard32_scale(const void* x, int bf16, int64_t rows, int64_t cols,
                                   int64_t ldx, const float* chan_scale, float* y, int64_t ldy,
                                   hipStream_t s) {
  const int64_t cpr = cols / 8, n = rows * cpr;
  const bool contig = (ldx == cols);
  const unsigned g = grid_for(n, kThreads);
  const bool sc = chan_scale != nullptr;
  if (bf16) {
    if (contig) launch_had_variant<true, true>(sc, g, s, x, n, cpr, ldx, chan_scale, y, ldy);
    else launch_had_variant<true, false>(sc, g, s, x, n, cpr, ldx, chan_scale, y, ldy);
  } else {
    if (contig) launch_had_variant<false, true>(sc, g, s, x, n, cpr, ldx, chan_scale, y, ldy);
    else launch_had_variant<false, false>(sc, g, s, x, n, cpr, ldx, chan_scale, y, ldy);
  }
  return hipGetLastError();
}

hipError_t launch_balance_scale(const void* w, int w_bf16, int64_t N, int64_t K, int64_t ldw,
                                const void* x, int x_bf16, int64_t M, int64_t ldx, double alpha,
                                float* t_out, float* u_out, hipStream_t s) {
  const unsigned g = grid_for(K, 64);
  if (w_bf16 && x_bf16) hipLaunchKernelGGL((k_balance<true, true>), dim3(g), dim3(kThreads), 0, s, w, N, K, ldw, x, M, ldx, alpha, t_out, u_out);
  else if (w_bf16) hipLaunchKernelGGL((k_balance<true, false>), dim3(g), dim3(kThreads), 0, s, w, N, K, ldw, x, M, ldx, alpha, t_out, u_out);
  else if (x_bf16) hipLaunchKernelGGL((k_balance<false, true>), dim3(g), dim3(kThreads), 0, s, w, N, K, ldw, x, M, ldx, alpha, t_out, u_out);
  else hipLaunchKernelGGL((k_balance<false, false>), dim3(g), dim3(kThreads), 0, s, w, N, K, ldw, x, M, ldx, alpha, t_out, u_out);
  return hipGetLastError();
}

hipError_t launch_sigma_delta(const fp4q_sd_segment* segs, int nseg, int steps,
                              int64_t bank_stride, int sched, int n_rtn, hipStream_t s) {
  for (int base = 0; base < nseg; base += kSdMaxSeg) {
    SdArgs a = {};
    const int cnt = (nseg - base) < kSdMaxSeg ? (nseg - base) : kSdMaxSeg;
    a.nseg = cnt;
    int32_t wg = 0;
    for (int i = 0; i < cnt; ++i) {
      const fp4q_sd_segment& g = segs[base + i];
      a.w[i] = g.w;
      a.scales[i] = g.scales;
      a.ts[i] = g.tensor_scale;
      a.res[i] = g.residue;
      a.codes[i] = g.codes;
      a.nchunks[i] = g.rows * (g.cols / 8);
      a.wg_start[i] = wg;
      wg += (int32_t)grid_for(a.nchunks[i], (int64_t)kThreads * kSdUnroll);
    }
    a.wg_start[cnt] = wg;
    if (sched) hipLaunchKernelGGL(k_sigma_delta<true>, dim3(wg), dim3(kThreads), 0, s, a, steps, bank_stride, n_rtn);
    else hipLaunchKernelGGL(k_sigma_delta<false>, dim3(wg), dim3(kThreads), 0, s, a, steps, bank_stride, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_harmonize_nvfp4(const fp4q_nv_member* mem, int n, float* shared, hipStream_t s) {
  HzArgs a = {};
  a.n = n;
  int32_t wg = 0;
  for (int i = 0; i < n; ++i) {
    a.scales[i] = mem[i].scales;
    a.ts[i] = mem[i].tensor_scale;
    a.nbytes[i] = mem[i].rows * (mem[i].cols / 16);
    const int64_t mis = (int64_t)(reinterpret_cast<uintptr_t>(mem[i].scales) & 15u);
    const int64_t head = mis ? 16 - mis : 0;
    a.head[i] = (int32_t)(head < a.nbytes[i] ? head : a.nbytes[i]);
    a.wg_start[i] = wg;
    const int64_t items = ((a.nbytes[i] - a.head[i]) >> 4) + 1;      // body chunks + the edge
    wg += (int32_t)grid_for(items, (int64_t)kThreads * kHzUnroll);
  }
  a.wg_start[n] = wg;
  hipLaunchKernelGGL(k_harmonize, dim3(wg), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_harmonize_cells, dim3(1), dim3(64), 0, s, a, shared);
  return hipGetLastError();
}

hipError_t launch_stochastic_round(const fp4q_sd_segment* segs, int nseg, int steps, int64_t bank_stride,
                                   uint64_t seed, uint32_t step0, int two_point, hipStream_t s) {
  for (int base = 0; base < nseg; base += kSdMaxSeg) {
    SdArgs a = {};
    const int cnt = (nseg - base) < kSdMaxSeg ? (nseg - base) : kSdMaxSeg;
    a.nseg = cnt;
    int32_t wg = 0;
    for (int i = 0; i < cnt; ++i) {
      const fp4q_sd_segment& g = segs[base + i];
      a.w[i] = g.w;
      a.scales[i] = g.scales;
      a.ts[i] = g.tensor_scale;
      a.res[i] = nullptr;
      a.codes[i] = g.codes;
      a.nchunks[i] = g.rows * (g.cols / 8);
      a.wg_start[i] = wg;
      wg += (int32_t)grid_for(a.nchunks[i], (int64_t)kThreads * kSdUnroll);
    }
    a.wg_start[cnt] = wg;
    if (two_point)
      hipLaunchKernelGGL(k_stochastic_round<true>, dim3(wg), dim3(kThreads), 0, s, a, steps, bank_stride, 0u, 0u,
                         step0, base);
    else
      hipLaunchKernelGGL(k_stochastic_round<false>, dim3(wg), dim3(kThreads), 0, s, a, steps, bank_stride,
                         (uint32_t)seed, (uint32_t)(seed >> 32), step0, base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4q
