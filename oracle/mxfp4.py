"""MXFP4 quantization, the per-channel balance scale and the block-32
Hadamard rotation.

Test infrastructure only (see ``oracle/__init__``).

Definitions followed ("MACaQ", paper 2611.10649):

* background box "MXFP4 micro-scaling format": OCP MXFP4, blocks of B = 32
  elements sharing one 8-bit pure-exponent E8M0 scale (a power of two),
  E2M1 elements, about 4.25 bits per element;
* "Core method", steps (i)-(ii) and "Method steps", steps 1-2: activations
  are multiplied by t_j per input channel, weight columns divided by t_j;
  then a block-32 orthogonal Hadamard B with +-1 entries is applied on the
  right, x' = (x * t) B and W' = (W / t) B; scaling happens BEFORE the
  rotation; the layer computes y = [(x*t)B]_MXFP4 [W']_MXFP4^T;
* "Method steps", step 3: the standard block exponent is derived from the
  block maximum; the OCP rule is floor(log2(amax)) - emax(E2M1), emax = 2.

Orthonormal block-32 Hadamard: Sylvester natural order H_32 (H_1 = [1],
H_2n = [[H, H], [H, -H]]) scaled by 1/sqrt(32).  Evaluated as the fast
transform with stages h = 1, 2, 4, 8, 16: for each pair (i, i+h) with
(i & h) == 0, (a, b) -> (a + b, a - b); then one multiplication of every
element by c = fl32(1/sqrt(32)).  Every add, subtract and multiply is one
binary32 operation.
"""

from __future__ import annotations

import numpy as np

from .formats import e2m1_round, e2m1_decode, e8m0_decode, floor_log2_f32

BLOCK = 32
F32 = np.float32
#: fl32(1/sqrt(32)) -- rounded once from the float64 value
HADAMARD_NORM = F32(1.0 / np.sqrt(np.float64(32.0)))


def fwht32_stages(z: np.ndarray) -> np.ndarray:
    """Unnormalised Sylvester-order fast Walsh-Hadamard transform of every
    aligned 32-block along the last axis, in binary32, stage order
    h = 1, 2, 4, 8, 16."""
    z = np.asarray(z, dtype=F32)
    R, K = z.shape
    assert K % BLOCK == 0
    y = z.reshape(R, K // BLOCK, BLOCK).copy()
    h = 1
    while h < BLOCK:
        for i in range(BLOCK):
            if i & h:
                continue
            a = y[..., i].copy()
            b = y[..., i + h].copy()
            y[..., i] = (a + b).astype(F32)
            y[..., i + h] = (a - b).astype(F32)
        h *= 2
    return y.reshape(R, K)


def hadamard32_scale(x: np.ndarray, chan_scale=None) -> np.ndarray:
    """y = fl(FWHT32(fl(x * t)) * c) for a float32 [R, K] tensor;
    ``chan_scale`` (float32 [K]) is t, or None for no balance scale."""
    x = np.asarray(x, dtype=F32)
    if chan_scale is not None:
        z = (x * np.asarray(chan_scale, dtype=F32)[None, :]).astype(F32)
    else:
        z = x
    return (fwht32_stages(z) * HADAMARD_NORM).astype(F32)


def quantize(y: np.ndarray):
    """MXFP4-quantize a float32 [R, K] tensor (K % 32 == 0).

    Returns ``(codes, scales)``: ``codes`` uint8 [R, K] unpacked 4-bit codes,
    ``scales`` uint8 [R, K/32] E8M0 bytes (= e + 127).

    Per block: a_b = max |y|; a_b == 0 -> byte 0x00 and codes 0x0; else
    e = floor(log2 a_b) - 2 clamped to [-127, 127]; v_i = fl(y_i * 2**-e);
    code_i = nearest E2M1 code (values in (6, 8) are nearest to 6).
    """
    y = np.asarray(y, dtype=F32)
    R, K = y.shape
    assert K % BLOCK == 0
    yb = y.reshape(R, K // BLOCK, BLOCK)
    a_b = np.abs(yb).max(axis=-1)
    nz = a_b > 0
    e = np.zeros(a_b.shape, dtype=np.int64)
    if nz.any():
        e[nz] = floor_log2_f32(a_b[nz]) - 2
    e = np.clip(e, -127, 127)
    e = np.where(nz, e, -127)
    inv = np.ldexp(np.float64(1.0), -e).astype(F32)          # 2**-e, exact in fp32
    v = (yb * inv[..., None]).astype(F32).reshape(R, K)
    codes = np.empty((R, K), dtype=np.uint8)
    for r0 in range(0, R, 256):
        codes[r0:r0 + 256] = e2m1_round(v[r0:r0 + 256])
    codes[np.repeat(~nz, BLOCK, axis=1)] = 0
    scales = (e + 127).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 value: value(code) * 2**(byte - 127)."""
    return e2m1_decode(codes) * np.repeat(e8m0_decode(scales), BLOCK, axis=1)
