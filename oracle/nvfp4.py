"""NVFP4 quantization and dequantization.

Test infrastructure only (see ``oracle/__init__``).

Definition followed:

* loopquant page, section 0.2: E2M1 elements, 16-element blocks, one E4M3
  block scale per block, one FP32 tensor scale; the decoded value of an
  element is code value x block scale x tensor scale.
* loopquant page, section 2.2 (paragraph applying the residue bound to the
  signed E2M1 code book): default tensor scale s_tensor = max|W| / (6*256);
  the candidate E4M3 block scale is rounded UP, which guarantees that the
  normalised value |x / s| is at most 6.
* "Why Gated DeltaNet Survives 4-Bit Quantization", background box "NVFP4
  and W4A4": the block scale is the block maximum / 6 (before the tensor
  scale is divided out); block max/RMS is at most 4 in a 16-element block.

* loopquant page, section 2.2 and the section 2.5 listing: the 4/6 block
  scaling (``rule="4/6"`` of :func:`quantize`).
* "Why Gated DeltaNet Survives 4-Bit Quantization", fused-GEMM global-scale
  box and pipeline step (2): one shared tensor scale for the members of a
  fused GEMM (:func:`harmonize`).

The order of the fp32 operations is the reading this project takes where the
pages are silent (recorded in the design notes): every step is a single
IEEE binary32 operation with round-to-nearest-even.

    A    = max |x| over the tensor                    (or a given s_t)
    s_t  = fl(A / 1536)                                 (0 if A == 0)
    a_b  = max |x_i| over the block
    s_b  = ceil_E4M3( fl(a_b / fl(6 * s_t)) )           (0 if a_b == 0 or s_t == 0)
    s    = fl(s_t * s_b);  rho = fl(1 / s)
    v_i  = fl(x_i * rho);  code_i = nearest E2M1 code of v_i
"""

from __future__ import annotations

import numpy as np

from .formats import e2m1_round, e2m1_decode, e4m3_ceil, e4m3_decode, e4m3_round_nearest

BLOCK = 16
F32 = np.float32


def tensor_scale_from_amax(amax) -> np.float32:
    """s_t = fl(A / (6*256)) in binary32 (loopquant page, section 2.2)."""
    a = F32(amax)
    return F32(a / F32(1536.0))


def block_scales(x: np.ndarray, s_t) -> np.ndarray:
    """E4M3 block-scale bytes for a float32 [R, K] tensor (K % 16 == 0)."""
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    assert K % BLOCK == 0
    s_t = F32(s_t)
    a_b = np.abs(x).reshape(R, K // BLOCK, BLOCK).max(axis=-1)       # exact
    six_st = F32(F32(6.0) * s_t)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (a_b / six_st).astype(F32)                                # fl32 division
    y = np.where((a_b == 0) | (s_t == 0), F32(0), y)
    return e4m3_ceil(y.astype(np.float64))


def _encode_with(x: np.ndarray, s_t, sb_bytes: np.ndarray):
    """Codes of ``x`` under the given block-scale bytes, and the decoded
    total scales s = fl(s_t * s_b) per block."""
    R, K = x.shape
    s_b = e4m3_decode(sb_bytes).astype(F32)                      # exact in fp32
    s = (F32(s_t) * s_b).astype(F32)                             # fl32 product
    with np.errstate(divide="ignore"):
        rho = (F32(1.0) / s).astype(F32)                         # fl32 reciprocal
    rho_e = np.repeat(rho, BLOCK, axis=1)
    with np.errstate(invalid="ignore"):                          # 0 * inf in zero blocks
        v = (x * rho_e).astype(F32)
    codes = np.empty((R, K), dtype=np.uint8)
    for r0 in range(0, R, 256):                                  # chunk to bound memory
        codes[r0:r0 + 256] = e2m1_round(v[r0:r0 + 256])
    zero_blk = np.repeat(s == 0, BLOCK, axis=1)
    codes[zero_blk] = 0
    return codes, s


def block_scales_to(x: np.ndarray, s_t, target) -> np.ndarray:
    """E4M3 block-scale bytes that map each block maximum to ``target`` (6
    or 4): ceil_E4M3(fl(a_b / fl(target * s_t)))."""
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    s_t = F32(s_t)
    a_b = np.abs(x).reshape(R, K // BLOCK, BLOCK).max(axis=-1)       # exact
    t_st = F32(F32(target) * s_t)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (a_b / t_st).astype(F32)                                  # fl32 division
    y = np.where((a_b == 0) | (s_t == 0), F32(0), y)
    return e4m3_ceil(y.astype(np.float64))


def block_sq_error(x: np.ndarray, codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Squared reconstruction error of every 16-block, in binary32, in this
    fixed order (the reading taken for the 4/6 choice; the pages give none):
        d_i = fl(x_i - fl(s * value(code_i))),  e_i = fl(d_i * d_i)
        T(h) = ((e0 + e1) + (e2 + e3)) + ((e4 + e5) + (e6 + e7))  per 8-element half
        E = fl(T(first half) + T(second half))"""
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    q = e2m1_decode(codes).astype(F32)                           # exact
    se = np.repeat(np.asarray(s, dtype=F32), BLOCK, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        d = (x - (se * q).astype(F32)).astype(F32)
        e = (d * d).astype(F32).reshape(R, K // BLOCK, 2, 8)
        p1 = (e[..., 0::2] + e[..., 1::2]).astype(F32)
        p2 = (p1[..., 0::2] + p1[..., 1::2]).astype(F32)
        t = (p2[..., 0] + p2[..., 1]).astype(F32)
        return (t[..., 0] + t[..., 1]).astype(F32)


def quantize(x: np.ndarray, tensor_scale=None, rule: str = "6"):
    """NVFP4-quantize a float32 [R, K] tensor.

    Returns ``(codes, scales, s_t)``: ``codes`` uint8 [R, K] (one 4-bit code
    per element, unpacked), ``scales`` uint8 [R, K/16] (E4M3 bytes),
    ``s_t`` float32.  With ``tensor_scale`` given it is used as s_t.

    ``rule="6"`` maps every block maximum to 6.  ``rule="4/6"`` is the 4/6
    block scaling of the loopquant page (section 2.2, residue-bound paragraph;
    ``block_scale_46`` in the section 2.5 listing): both candidate scales,
    block maximum to 6 and to 4, keep |x / s| <= 6, and each block takes the
    one with the smaller squared error (:func:`block_sq_error`); ties go to 6.
    """
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    if tensor_scale is None:
        s_t = tensor_scale_from_amax(np.abs(x).max() if x.size else F32(0))
    else:
        s_t = F32(tensor_scale)
    sb6 = block_scales(x, s_t)
    codes6, s6 = _encode_with(x, s_t, sb6)
    if rule == "6":
        return codes6, sb6, s_t
    assert rule == "4/6", rule
    sb4 = block_scales_to(x, s_t, 4)
    codes4, s4 = _encode_with(x, s_t, sb4)
    pick4 = block_sq_error(x, codes4, s4) < block_sq_error(x, codes6, s6)   # ties: 6
    sb = np.where(pick4, sb4, sb6).astype(np.uint8)
    codes = np.where(np.repeat(pick4, BLOCK, axis=1), codes4, codes6).astype(np.uint8)
    return codes, sb, s_t


def dequantize(codes: np.ndarray, scales: np.ndarray, s_t) -> np.ndarray:
    """Exact float64 value of every element: value(code) * s_b * s_t
    (at most 2 + 4 + 24 significant bits, so float64 holds it exactly)."""
    q = e2m1_decode(codes)
    sb = np.repeat(e4m3_decode(scales), BLOCK, axis=1)
    return q * sb * np.float64(F32(s_t))


def harmonize(scales, tensor_scales):
    """One shared tensor scale for the members of a fused projection.

    "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
    Recurrent Half of a Hybrid 27B LLM", background box on fused GEMMs and
    the global-scale mismatch, and step (2) of its pipeline: the members of a
    fused NVFP4 GEMM are rewritten to one shared global scale (the largest
    member scale, the one the fused GEMM uses), each member's ratio folded
    into its E4M3 block scales; codes are unchanged and the re-rounding is at
    most half an E4M3 step (the page reports <= 6.2%).  Reading: the scale is
    the decode multiplier s_t of this module, so every ratio is <= 1 and no
    block scale can pass 448; a block scale that falls below half the
    smallest E4M3 subnormal becomes 0.
        s_t  = max_i s_t,i
        r_i  = fl(s_t,i / s_t)                 (1 if s_t == 0)
        s_b' = nearest_E4M3( fl(s_b * r_i) )   (ties to even)
    Bytes that are not a non-negative finite E4M3 value (sign bit set, or
    NaN), which no quantizer here writes, are left as they are.  After the
    rewrite every member decodes with s_t.
    Returns (list of new scale-byte arrays, s_t)."""
    sts = [F32(t) for t in tensor_scales]
    st = max(sts)
    out = []
    for sb, ti in zip(scales, sts):
        sb = np.asarray(sb, dtype=np.uint8)
        r = F32(ti / st) if st > 0 else F32(1.0)
        valid = sb <= 0x7E
        dec = e4m3_decode(np.where(valid, sb, 0).astype(np.uint8)).astype(F32)
        prod = (dec * r).astype(F32)
        out.append(np.where(valid, e4m3_round_nearest(prod.astype(np.float64)), sb).astype(np.uint8))
    return out, st
