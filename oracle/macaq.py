"""MACaQ weight-side refinement of an MXFP4 weight: input Hessian, ridge,
Hessian-weighted E8M0 exponent screen and Flip-Refinement.

Test infrastructure only (see ``oracle/__init__``).

Definition followed: "MACaQ: Fast, Model Agnostic Calibrated Quantization
for Low-Precision Weights and Activations", "Core method" steps (iii) and
(iv) and "Method steps" 0, 3 and 4 (Algorithm 1, equations 12 and 15):

* calibration: H = sum over calibration tokens of x^T x, in the domain of
  the transformed weight W' (the inputs here are already scaled and
  rotated);
* ridge: H_f = H + lambda * mean(diag H) * I, lambda = 1.0;
* exponent screen: for each row and 32-element block, among the standard
  exponent e0 (from the block maximum, as the MXFP4 quantizer takes it) and
  e0 + 1, e0 - 1, keep the one minimising
  E(e) = sum_j (H_f)_jj (W'_ij - What_ij(e))^2, What(e) the nearest-code
  quantization at scale 2^e; the exponents then stay fixed;
* Flip-Refinement: start from those codes; with r_i = W'_i - What_i and
  g_i = r_i H_f, a move of code (i, j) to an adjacent E2M1 grid point that
  changes What_ij by D lowers the row objective r_i H_f r_i^T by
  gain = 2 D g_ij - D^2 (H_f)_jj; each round every active row takes its
  largest positive gain and updates g_i <- g_i - D (H_f)_{j,:}; a row
  without a positive gain leaves the active set; at most K rounds.

Readings (the page fixes neither precision nor order; recorded in the
design notes):

* float64 throughout.  Every sum runs in a fixed sequential order:
  H_jk over tokens in order; sum diag H over j; the block error over the
  32 elements in order; g_ij over k in order.  Products of two float32 are
  exact in float64; a step D is a power of two, so D * g, D * D * H_jj and
  D * H_jk are exact and every gain or update is a single rounding.
* Ties: the screen keeps e0 unless a candidate is strictly better, trying
  e0 + 1 before e0 - 1; candidates outside [-127, 127] are skipped.  A flip
  takes the first maximum in the order (j ascending, the move down before
  the move up).
* A value of 0 is written as code 0x8 when W'_ij has its sign bit set,
  else 0x0 (the sign rule of the nearest-code quantizer).  An all-zero
  block keeps scale byte 0x00 and codes 0x0 and is never flipped.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_VALUES, e2m1_round, floor_log2_f32

F32 = np.float32
F64 = np.float64
BLOCK = 32
#: the 15 distinct E2M1 values in increasing order (the flip grid)
GRID = np.array([-6.0, -4.0, -3.0, -2.0, -1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
ZERO_INDEX = 7


def hessian(x: np.ndarray, h: np.ndarray | None = None) -> np.ndarray:
    """h + sum_t x_t^T x_t for float32 x [T, n], float64, tokens in order."""
    x = np.asarray(x, dtype=F32).astype(F64)
    n = x.shape[1]
    h = np.zeros((n, n), F64) if h is None else np.array(h, dtype=F64)
    for t in range(x.shape[0]):
        h += np.outer(x[t], x[t])                 # exact products, one rounding per add
    return h


def ridge_delta(h: np.ndarray, lam: float = 1.0) -> F64:
    """lambda * mean(diag h): the sum over j in order, then / n, then * lambda."""
    s = F64(0.0)
    for v in np.diag(h):
        s = F64(s + v)
    return F64(F64(lam) * F64(s / F64(h.shape[0])))


def ridged_diag(h: np.ndarray, delta) -> np.ndarray:
    return (np.diag(h).astype(F64) + F64(delta)).astype(F64)


def _code_values(codes: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[codes & 0xF]


def _encode_at(wb: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Nearest codes of the float32 blocks wb [..., 32] at scale 2^e."""
    inv = np.ldexp(F64(1.0), -e).astype(F32)     # 2^-e, exact in float32
    return e2m1_round((wb * inv[..., None]).astype(F32))


def _block_error(wb: np.ndarray, codes: np.ndarray, e: np.ndarray, hd: np.ndarray) -> np.ndarray:
    """sum_j hd_j * (w_j - value_j * 2^e)^2 over each block, in order."""
    what = _code_values(codes) * np.ldexp(F64(1.0), e)[..., None]
    d = wb.astype(F64) - what                    # exact
    t = hd.reshape(1, -1, BLOCK) * (d * d)
    err = np.zeros(wb.shape[:-1], F64)
    for j in range(BLOCK):
        err = err + t[..., j]
    return err


def screen(w: np.ndarray, hd: np.ndarray):
    """Exponent screen.  w float32 [m, n] (n % 32 == 0), hd = diag(H_f)
    float64 [n].  Returns (codes uint8 [m, n] unpacked, exponents int64
    [m, n/32], all-zero-block mask [m, n/32])."""
    w = np.asarray(w, dtype=F32)
    m, n = w.shape
    wb = w.reshape(m, n // BLOCK, BLOCK)
    a = np.abs(wb).max(axis=-1)
    nz = a > 0
    e0 = np.full(a.shape, -127, np.int64)
    if nz.any():
        e0[nz] = np.clip(floor_log2_f32(a[nz]) - 2, -127, 127)
    best_e = e0.copy()
    best_c = _encode_at(wb, e0)
    best_err = _block_error(wb, best_c, e0, hd)
    for off in (1, -1):
        ec = e0 + off
        ok = nz & (ec >= -127) & (ec <= 127)
        ecs = np.clip(ec, -127, 127)
        c = _encode_at(wb, ecs)
        err = _block_error(wb, c, ecs, hd)
        better = ok & (err < best_err)
        best_e = np.where(better, ecs, best_e)
        best_err = np.where(better, err, best_err)
        best_c = np.where(better[..., None], c, best_c)
    best_c[~nz] = 0
    return best_c.reshape(m, n), best_e, ~nz


def gradient(w: np.ndarray, codes: np.ndarray, e: np.ndarray, h: np.ndarray, delta) -> np.ndarray:
    """g = r H_f with r = w - What, each g_ij summed over k in order."""
    w = np.asarray(w, dtype=F32)
    m, n = w.shape
    what = _code_values(codes) * np.repeat(np.ldexp(F64(1.0), e), BLOCK, axis=1)
    r = w.astype(F64) - what
    hf = np.array(h, dtype=F64)
    hf[np.arange(n), np.arange(n)] = ridged_diag(h, delta)
    g = np.zeros((m, n), F64)
    for k in range(n):
        g = g + r[:, k:k + 1] * hf[k][None, :]   # product rounded, then the add
    return g


def _grid_index(codes: np.ndarray) -> np.ndarray:
    return np.searchsorted(GRID, _code_values(codes))


def flip_refine(w, codes, e, zero_blocks, h, delta, k_iters: int = 128, g=None):
    """Flip-Refinement from the given codes at fixed exponents.  Returns
    (codes uint8 [m, n] unpacked, flips per row int64 [m])."""
    w = np.asarray(w, dtype=F32)
    m, n = w.shape
    g = gradient(w, codes, e, h, delta) if g is None else np.array(g, dtype=F64)
    hf = np.array(h, dtype=F64)
    hd = ridged_diag(h, delta)
    hf[np.arange(n), np.arange(n)] = hd
    idx = _grid_index(codes)
    scale = np.repeat(np.ldexp(F64(1.0), e), BLOCK, axis=1)
    frozen = np.repeat(zero_blocks, BLOCK, axis=1)
    rows = np.arange(m)
    active = np.ones(m, bool)
    flips = np.zeros(m, np.int64)
    for _ in range(k_iters):
        gains = np.full((m, n, 2), -np.inf)
        for k, step in ((0, -1), (1, 1)):
            nxt = idx + step
            ok = (nxt >= 0) & (nxt < GRID.size) & ~frozen
            d = (GRID[np.clip(nxt, 0, GRID.size - 1)] - GRID[idx]) * scale    # exact power of two
            gain = (2.0 * d) * g - (d * d) * hd[None, :]
            gains[..., k] = np.where(ok, gain, -np.inf)
        flat = gains.reshape(m, 2 * n)
        best = flat.argmax(axis=1)                 # first maximum
        take = active & (flat[rows, best] > 0)
        if not take.any():
            break
        for i in np.nonzero(take)[0]:
            j, k = divmod(int(best[i]), 2)
            step = -1 if k == 0 else 1
            d = (GRID[idx[i, j] + step] - GRID[idx[i, j]]) * scale[i, j]
            idx[i, j] += step
            g[i] = g[i] - d * hf[j]
        flips += take
        active = take
    vals = GRID[idx]
    mag = np.searchsorted(E2M1_VALUES[:8], np.abs(vals)).astype(np.uint8)
    neg = (vals < 0) | ((vals == 0) & np.signbit(w))
    out = mag | (neg.astype(np.uint8) << 3)
    out[frozen] = 0
    return out, flips


def refine(w: np.ndarray, h: np.ndarray, lam: float = 1.0, k_iters: int = 128):
    """The whole weight-side refinement.  Returns (codes uint8 [m, n]
    unpacked, E8M0 scale bytes uint8 [m, n/32], flips per row)."""
    delta = ridge_delta(h, lam)
    codes, e, zb = screen(w, ridged_diag(h, delta))
    if k_iters > 0:
        codes, flips = flip_refine(w, codes, e, zb, h, delta, k_iters)
    else:
        flips = np.zeros(np.asarray(w).shape[0], np.int64)
    return codes, (e + 127).astype(np.uint8), flips


def objective(w: np.ndarray, codes: np.ndarray, scales: np.ndarray, hf: np.ndarray) -> np.ndarray:
    """r_i H_f r_i^T per row, float64 (for checks; no fixed order)."""
    what = _code_values(codes) * np.repeat(np.ldexp(F64(1.0), scales.astype(np.int64) - 127), BLOCK, axis=1)
    r = np.asarray(w, F32).astype(F64) - what
    return np.einsum("ij,jk,ik->i", r, hf, r)
