"""GEMM oracle over exactly dequantized operands.

Test infrastructure only (see ``oracle/__init__``).

The layer the pages describe multiplies quantized activations by quantized
weights, y = x_hat W_hat^T ("MACaQ", "Core method": y = [(x*t)B]_MXFP4
W'^T_MXFP4; "Why Gated DeltaNet Survives 4-Bit Quantization", background box
"NVFP4 and W4A4": both operands in NVFP4).  Fake quantization -- quantize,
dequantize, compute in high precision -- is the semantics the GDN paper uses
for its error studies ("Core method").  The oracle is exactly that: dequantize
both operands exactly (float64 holds every NVFP4 / MXFP4 / bf16 value
exactly) and multiply in float64 (NumPy matmul as the library primitive).
"""

from __future__ import annotations

import numpy as np

from . import nvfp4, mxfp4
from .formats import bf16_bits_to_f32


def matmul_nt(a64: np.ndarray, b64: np.ndarray) -> np.ndarray:
    """Y = A B^T in float64 (A [M, K], B [N, K])."""
    return np.asarray(a64, np.float64) @ np.asarray(b64, np.float64).T


def w4a4_nvfp4(a_codes, a_scales, a_st, b_codes, b_scales, b_st) -> np.ndarray:
    return matmul_nt(nvfp4.dequantize(a_codes, a_scales, a_st),
                     nvfp4.dequantize(b_codes, b_scales, b_st))


def w4a4_mxfp4(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    return matmul_nt(mxfp4.dequantize(a_codes, a_scales),
                     mxfp4.dequantize(b_codes, b_scales))


def w4a16(a_bf16_bits, b_codes, b_scales, b_st) -> np.ndarray:
    """bf16 activations (uint16 bit patterns) times an NVFP4 weight."""
    a = bf16_bits_to_f32(a_bf16_bits).astype(np.float64)
    return matmul_nt(a, nvfp4.dequantize(b_codes, b_scales, b_st))


def rel_err(y, y_ref):
    """(whole-matrix Frobenius relative error, worst per-row relative error,
    max|dy| / max|y_ref|).  Rows whose reference is all zero count their
    absolute error relative to the whole-matrix norm."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    d = y - y_ref
    nref = np.linalg.norm(y_ref)
    whole = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    row_ref = np.linalg.norm(y_ref, axis=1)
    row_d = np.linalg.norm(d, axis=1)
    denom = np.where(row_ref > 0, row_ref, nref if nref > 0 else 1.0)
    worst_row = float((row_d / denom).max()) if y.size else 0.0
    mref = np.abs(y_ref).max() if y.size else 0.0
    maxrel = float(np.abs(d).max() / mref) if mref > 0 else float(np.abs(d).max() if y.size else 0.0)
    return float(whole), worst_row, maxrel
