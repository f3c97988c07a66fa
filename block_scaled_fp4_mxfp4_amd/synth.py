"""Seeded synthetic inputs for the five workloads.

This module holds input generation only -- no quantization, scaling,
rotation or GEMM arithmetic -- so that both the HIP path and the CPU oracle
can consume the same bytes.  It imports neither of them.

Recipe (numpy PCG64 via ``default_rng``):

* values: ``standard_normal`` in float64, times sigma, rounded to float32
  (round-to-nearest-even), then to bf16 (round-to-nearest-even on the fp32
  bit pattern) where the workload is bf16;
* heavy-tailed activations stand in for the captured LLM activations of the
  GDN study ("Why Gated DeltaNet Survives 4-Bit Quantization": median-layer
  row max/RMS 63.5, kurtosis about 1564, 10-32 % of 16-blocks dominated by
  one value): N(0, 1) with 1 % of the input channels (columns) chosen by a
  second seeded generator and multiplied by 64;
* weights: N(0, 0.02**2).

bf16 tensors are returned as uint16 bit patterns (NumPy has no bf16).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) -> uint16 bit patterns.
    Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


def uint8_bytes(seed: int, shape, lo: int = 0, hi: int = 256) -> np.ndarray:
    """Uniform random bytes in [lo, hi)."""
    return np.random.default_rng(seed).integers(lo, hi, shape, dtype=np.uint8)


def outlier_columns(seed: int, k: int, count: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(k, size=count, replace=False))


def heavy_tailed_f32(seed: int, col_seed: int, shape, frac: float = 0.01,
                     factor: float = 64.0, count: int = None) -> np.ndarray:
    """N(0,1) [rows, K] with round(frac*K) (or ``count``) columns times ``factor``."""
    rows, k = shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k))
    n_out = int(round(frac * k)) if count is None else int(count)
    cols = outlier_columns(col_seed, k, n_out)
    x[:, cols] *= factor
    return x.astype(np.float32)


# ------------------------------------------------------------ workloads ----

#: the looped-core linears: 13 linears cycling q, k, v, o (768x768),
#: gate, up (3072x768) and down (768x3072) -- [N, K] = [out, in]
LOOPED_SHAPES: List[Tuple[int, int]] = [
    (768, 768), (768, 768), (768, 768), (768, 768),
    (3072, 768), (3072, 768), (768, 3072),
    (768, 768), (768, 768), (768, 768), (768, 768),
    (3072, 768), (3072, 768),
]


# Workload seeds: seed 0 is the default input set; seed s adds
# SEED_STRIDE * s to every generator seed of the workload.
SEED_STRIDE = 100_000


@dataclass
class Workload:
    name: str
    arrays: Dict[str, np.ndarray] = field(default_factory=dict)
    meta: Dict[str, object] = field(default_factory=dict)


def nvfp4_tiny(seed: int = 0) -> Workload:
    """NVFP4 W4A4 linear, tiny: X fp32 [64x256] N(0,1) with 2 outlier
    channels x50; W fp32 [256x256] N(0, 0.02**2)."""
    o = SEED_STRIDE * seed
    x = heavy_tailed_f32(1001 + o, 1003 + o, (64, 256), count=2, factor=50.0)
    w = normal_f32(1002 + o, (256, 256), 0.02)
    return Workload("nvfp4_tiny_64x256x256", {"x": x, "w": w},
                    {"M": 64, "N": 256, "K": 256})


def nvfp4_prefill(m: int = 4096, n: int = 10240, k: int = 5120, seed: int = 0) -> Workload:
    """NVFP4 prefill linear: X bf16 [4096x5120] heavy-tailed; W bf16
    generated as [K x N] = [5120x10240] N(0, 0.02**2) and stored [N x K]."""
    o = SEED_STRIDE * seed
    x = f32_to_bf16_bits(heavy_tailed_f32(2001 + o, 2003 + o, (m, k)))
    w_kn = normal_f32(2002 + o, (k, n), 0.02)
    w = f32_to_bf16_bits(np.ascontiguousarray(w_kn.T))
    return Workload(f"nvfp4_prefill_{m}x{n}x{k}", {"x_bf16": x, "w_bf16": w},
                    {"M": m, "N": n, "K": k})


def mxfp4_transform(m: int = 2048, n: int = 14336, k: int = 4096, seed: int = 0) -> Workload:
    """MXFP4 linear with online transform: X bf16 [2048x4096] heavy-tailed,
    W bf16 [14336x4096] N(0, 0.02**2)."""
    o = SEED_STRIDE * seed
    x = f32_to_bf16_bits(heavy_tailed_f32(3001 + o, 3003 + o, (m, k)))
    w = f32_to_bf16_bits(normal_f32(3002 + o, (n, k), 0.02))
    return Workload(f"mxfp4_transform_{m}x{n}x{k}", {"x_bf16": x, "w_bf16": w},
                    {"M": m, "N": n, "K": k})


def nvfp4_decode(n: int = 17408, k: int = 5120, m_max: int = 16, seed: int = 0) -> Workload:
    """NVFP4 decode: X bf16 [16x5120] heavy-tailed (the first M rows are
    used, M in {1, 4, 16}); W fp32 [17408x5120] N(0, 0.02**2), quantized
    once outside the timed region."""
    o = SEED_STRIDE * seed
    x = f32_to_bf16_bits(heavy_tailed_f32(4001 + o, 4003 + o, (m_max, k)))
    w = normal_f32(4002 + o, (n, k), 0.02)
    return Workload(f"nvfp4_decode_{n}x{k}", {"x_bf16": x, "w": w},
                    {"N": n, "K": k, "M_list": [1, 4, 16]})


def looped_sigma_delta(tokens: int = 4096, seed: int = 0) -> Workload:
    """Looped core: 13 fp32 masters N(0, 0.02**2) (seed 5002 + 10 i), hidden
    state bf16 [8x512x768] = [4096x768] heavy-tailed, and a [4096x3072]
    heavy-tailed bf16 input for the down projection; R = 32 steps."""
    o = SEED_STRIDE * seed
    arrays = {}
    for i, (n, k) in enumerate(LOOPED_SHAPES):
        arrays[f"w{i}"] = normal_f32(5002 + 10 * i + o, (n, k), 0.02)
    arrays["h_bf16"] = f32_to_bf16_bits(heavy_tailed_f32(5001 + o, 5003 + o, (tokens, 768)))
    arrays["hd_bf16"] = f32_to_bf16_bits(heavy_tailed_f32(5011 + o, 5013 + o, (tokens, 3072)))
    return Workload("looped_sigma_delta_13x_R32", arrays,
                    {"R": 32, "tokens": tokens, "shapes": LOOPED_SHAPES})


def realized_stats(x: np.ndarray) -> Dict[str, float]:
    """Statistics of an activation tensor that the generator is meant to
    reproduce (row max/RMS, kurtosis, one-hot block fractions).  A block is
    one-hot when one value holds more than half of the block's energy."""
    x = np.asarray(x, dtype=np.float64)
    rms = np.sqrt((x * x).mean(axis=1))
    ratio = np.abs(x).max(axis=1) / rms
    xc = x - x.mean()
    kurt = float((xc ** 4).mean() / (xc ** 2).mean() ** 2)
    out = {"row_max_over_rms_median": float(np.median(ratio)),
           "row_max_over_rms_max": float(ratio.max()), "kurtosis": kurt}
    for b in (16, 32):
        e = (x * x).reshape(x.shape[0], -1, b)
        tot = e.sum(axis=-1)
        out[f"one_hot_frac_{b}"] = float((e.max(axis=-1) > 0.5 * tot).mean())
    return out
