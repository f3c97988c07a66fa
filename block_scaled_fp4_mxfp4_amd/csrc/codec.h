// codec.h -- device-side number formats for libfp4q (gfx950).
//
// E2M1 (FP4): sign, 2-bit exponent (bias 1), 1-bit mantissa; magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}; 16 codes, 15 values ("Looped Transformer
// quantization ...", section 0.2; end points +-6 and gap 2 in section 2.2).
// E4M3 (OCP E4M3FN): bias 7, subnormals, max 448, 0x7F NaN -- the NVFP4
// block scale ("Why Gated DeltaNet Survives 4-Bit Quantization", box
// "NVFP4 and W4A4").  E8M0: pure power-of-two exponent, the MXFP4 block
// scale ("MACaQ", box "MXFP4 micro-scaling format").
//
// Every function here is exact or a single correctly rounded binary32
// operation; translation units including it are built with
// -ffp-contract=off so that no multiply-add is fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// ---------------------------------------------------------------- E2M1 ----

// Nearest E2M1 magnitude index of |v|, ties to the even index (the OCP
// round-half-to-even rule), saturating above 6.  Decision points are the
// midpoints between neighbours; at a midpoint the comparison goes to the
// even side, hence the alternating > / >=.  NaN maps to 0.
__device__ __forceinline__ uint32_t e2m1_mag_index(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t i = (a > 0.25f);
  i += (a >= 0.75f);
  i += (a > 1.25f);
  i += (a >= 1.75f);
  i += (a > 2.5f);
  i += (a >= 3.5f);
  i += (a > 5.0f);
  return i;
}

// Full 4-bit code: sign bit (bit 3) = sign bit of v.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  return e2m1_mag_index(v) | ((__float_as_uint(v) >> 28) & 0x8u);
}

// Exact binary32 value of a 4-bit code (built from the bit fields).
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  bits |= (c & 8u) << 28;
  return __uint_as_float(bits);
}

// ---------------------------------------------------------------- E4M3 ----

// Smallest non-negative finite E4M3 value >= y (y finite, >= 0), as a byte;
// values above 448 give 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_ceil(float y) {
  if (!(y > 0.0f)) return 0u;
  if (y > 448.0f) return 0x7Eu;
  if (y < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
    const float t = y * 512.0f;              // exact (power-of-two scaling)
    uint32_t m = (uint32_t)t;                // floor, t in (0, 8)
    if ((float)m < t) ++m;                   // ceil; m == 8 is 2^-6 = byte 0x08
    return m;
  }
  const uint32_t b = __float_as_uint(y);
  int32_t e = (int32_t)((b >> 23) & 0xFFu) - 127;   // in [-6, 8]
  uint32_t q = (b >> 20) & 7u;
  if (b & 0xFFFFFu) ++q;
  if (q == 8u) { q = 0u; ++e; }
  return ((uint32_t)(e + 7) << 3) | q;       // y <= 448 keeps this <= 0x7E
}

// Exact binary32 value of a non-negative E4M3 byte (0x00..0x7E).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  if (e == 0u) return (float)m * 0.001953125f;           // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Nearest E4M3 byte to a binary32 f in [0, 448], ties to the even byte.
// Below 2^-6 the E4M3 grid is m * 2^-9 (m = 0..8; m = 8 is byte 0x08, the
// smallest normal), so the byte is the integer nearest to f * 2^9.  Above,
// the three leading mantissa bits are rounded to nearest-even on the
// binary32 pattern; a carry moves into the exponent field, and the exponent
// bias changes from 127 to 7 (120 << 3 = 960 in byte units).
__device__ __forceinline__ uint32_t e4m3_round_nearest(float f) {
  if (f < 0.015625f) return (uint32_t)__builtin_rintf(f * 512.0f);
  const uint32_t u = __float_as_uint(f);
  return ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;
}

// ---------------------------------------------------------------- E8M0 ----

// MXFP4 block exponent e = floor(log2 a) - 2 clamped to [-127, 127] for a
// finite a > 0, from the binary32 bit pattern (subnormals via the leading
// zero count).  Returns e; the scale byte is e + 127.
__device__ __forceinline__ int32_t mx_block_exponent(float a) {
  const uint32_t b = __float_as_uint(a);
  const uint32_t be = (b >> 23) & 0xFFu;
  int32_t fl;
  if (be) {
    fl = (int32_t)be - 127;
  } else {
    const uint32_t m = b & 0x7FFFFFu;       // non-zero for a > 0
    fl = -127 - (int32_t)(__builtin_clz(m) - 9);  // m * 2^-149, msb at 31-clz
  }
  int32_t e = fl - 2;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

// 2^-e as binary32 for e in [-127, 127] (always a normal number).
__device__ __forceinline__ float pow2_neg(int32_t e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// ---------------------------------------------------------------- misc ----

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

}  // namespace fp4q
