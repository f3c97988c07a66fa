"""Element and scale formats: E2M1 (FP4), E4M3 (FP8 block scale of NVFP4),
E8M0 (power-of-two block scale of MXFP4), and bf16 widening.

Test infrastructure only (see ``oracle/__init__``).

Sources (titles of the pages; sections as they appear there):

* "Looped Transformer quantization: error propagation, NVFP4 and Sigma-Delta
  modulation" (mer.dev, loopquant-fp4), section 0.2 "NVFP4 precision split":
  E2M1 has one sign, two exponent and one mantissa bit; eight non-negative
  grid points; sixteen codes but fifteen distinct values because +0 and -0
  coincide.  Section 2.2 gives the signed E2M1 end points [-6, 6] and the
  largest neighbour gap d = 2.
* "Why Gated DeltaNet Survives 4-Bit Quantization" (paper 2609.04098),
  background box "NVFP4 and W4A4": E2M1 elements, one E4M3 scale per 16
  elements, one FP32 tensor scale.
* "MACaQ" (paper 2611.10649), background box "MXFP4 micro-scaling format":
  OCP MXFP4, blocks of 32, an 8-bit pure-exponent E8M0 power-of-two scale.

E2M1 bit layout (OCP): code = s e1 e0 m, exponent bias 1.  Exponent field 0
is the subnormal range m * 0.5; otherwise 2**(e-1) * (1 + m/2).  This makes
the non-negative grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

E4M3 is the OCP "E4M3FN" flavour: bias 7, subnormals m/8 * 2**-6, no
infinities, 0x7F / 0xFF are NaN, largest finite value 448.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------- E2M1 ----

def e2m1_decode_scalar(code: int) -> float:
    """Value of one 4-bit E2M1 code from its bit fields (sign, 2-bit
    exponent with bias 1, 1-bit mantissa), as defined in the loopquant page
    section 0.2 and the OCP FP4 layout it names."""
    code = int(code) & 0xF
    s = code >> 3
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return -mag if s else mag


#: value of each of the 16 codes, indexed by code (float64, exact)
E2M1_VALUES = np.array([e2m1_decode_scalar(c) for c in range(16)], dtype=np.float64)
#: the eight non-negative magnitudes, indexed by the 3-bit magnitude index
E2M1_MAGNITUDES = E2M1_VALUES[:8].copy()


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of 4-bit codes (uint8 array, one code per element)
    to float64."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each float32 value ``v``.

    The definition (loopquant page, sections 2.1-2.2 and the STE listing of
    section 2.5: "take the nearest E2M1 code", a quantizer that saturates to
    the end points outside the hull): for |v| pick the nearest of the eight
    magnitudes; exact ties go to the magnitude with an even index (mantissa
    bit 0, the IEEE round-to-nearest-even rule the OCP conversion uses); the
    sign bit of the code is the sign bit of ``v`` (so -0.1 -> 0x8).  Values
    beyond 6 are nearest to 6, which is the saturation.

    Evaluated by comparing |v| with every magnitude in float64, not by a
    threshold table.  |v| is first clamped to 16: every value above 6 has 6
    as its nearest point, so the clamp cannot change the choice, and below
    16 the float64 differences |v| - m are exact for float32 |v| >= 2**-20
    (smaller |v| are nearest to 0 by a margin no rounding can close).
    """
    v = np.asarray(v, dtype=np.float32)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    idx = np.arange(8)
    for c0 in range(0, flat.size, 1 << 20):                  # bound temporaries
        vc = flat[c0:c0 + (1 << 20)]
        a = np.minimum(np.abs(vc.astype(np.float64)), 16.0)
        dist = np.abs(a[:, None] - E2M1_MAGNITUDES)            # [n, 8], exact
        is_min = dist == dist.min(axis=1, keepdims=True)
        # among the minimal candidates (one, or two on an exact tie) prefer
        # the even index
        even_pref = np.where(is_min & (idx % 2 == 0), idx, 99).min(axis=1)
        any_pref = np.where(is_min, idx, 99).min(axis=1)
        mag = np.where(even_pref < 99, even_pref, any_pref).astype(np.uint8)
        out[c0:c0 + vc.size] = mag | (np.signbit(vc).astype(np.uint8) << 3)
    return out.reshape(v.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes two per byte along the last axis: element 2j in the
    low nibble of byte j, element 2j+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ---------------------------------------------------------------- E4M3 ----

def e4m3_decode_scalar(byte: int) -> float:
    """Value of one OCP E4M3FN byte (bias 7, subnormals, no Inf, S.1111.111
    is NaN)."""
    byte = int(byte) & 0xFF
    s = byte >> 7
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


#: value of every byte 0..255 (float64; NaN at 0x7F and 0xFF)
E4M3_VALUES = np.array([e4m3_decode_scalar(b) for b in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_decode(bytes_: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(bytes_, dtype=np.uint8)]


def e4m3_ceil(y: np.ndarray) -> np.ndarray:
    """Smallest non-negative finite E4M3 value >= y, as a byte.

    The NVFP4 block scale is "rounded up" to E4M3 (loopquant page, section
    2.2, the paragraph applying the bound to the signed E2M1 code book).
    Values above 448 (including +inf) saturate to 448 (byte 0x7E); y == 0
    gives 0.
    Brute force over the 127 non-negative finite codes 0x00..0x7E, which are
    in increasing order of value.
    """
    y = np.asarray(y, dtype=np.float64)
    assert not np.any(np.isnan(y)) and np.all(y >= 0)
    table = E4M3_VALUES[:127]                      # 0x00 .. 0x7E, increasing
    assert np.all(np.diff(table) > 0)
    idx = np.searchsorted(table, y, side="left")   # first table[i] >= y
    idx = np.minimum(idx, 126)
    return idx.astype(np.uint8)


def e4m3_round_nearest(y: np.ndarray) -> np.ndarray:
    """Nearest non-negative finite E4M3 value to y (y >= 0), as a byte; ties
    go to the even byte (even mantissa); above 448 saturates to 448 (0x7E).
    Brute force over the 127 non-negative finite codes, like
    :func:`e4m3_ceil`."""
    y = np.asarray(y, dtype=np.float64)
    assert not np.any(np.isnan(y)) and np.all(y >= 0)
    table = E4M3_VALUES[:127]
    hi = np.minimum(np.searchsorted(table, y, side="left"), 126)   # first table[i] >= y
    lo = np.maximum(hi - 1, 0)
    d_hi = table[hi] - y
    d_lo = y - table[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    out = np.where(pick_lo & (hi > 0) & (y < table[126]), lo, hi)
    return out.astype(np.uint8)


# ---------------------------------------------------------------- E8M0 ----

def e8m0_decode(bytes_: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2**(byte-127) (0xFF is NaN)."""
    b = np.asarray(bytes_, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 255, np.nan, out)


def floor_log2_f32(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for positive float32 ``a`` (normal or subnormal), exact,
    via frexp on the exactly widened value: a = f * 2**x with f in [0.5, 1)."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    assert np.all(a > 0)
    _, x = np.frexp(a)
    return (x - 1).astype(np.int64)


# ---------------------------------------------------------------- bf16 ----

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 (held as uint16 bit patterns) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ------------------------------------------------------- exact helpers ----

def e2m1_values_fraction():
    """The 16 code values as exact Fractions (for the rational-mode tests)."""
    return [Fraction(float(E2M1_VALUES[c])) for c in range(16)]
