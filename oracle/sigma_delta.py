"""First-order Sigma-Delta weight re-quantization across loop steps.

Test infrastructure only (see ``oracle/__init__``).

Definition (loopquant page, section 2.1 "First-order Sigma-Delta", section
2.2 "Conservative residue bound on the non-uniform NVFP4 code book" and the
STE listing of section 2.5): with a FIXED scale and r_0 = 0, at each access
k = 1..R

    v_k = x + r_{k-1};   q_k = Q(v_k);   r_k = v_k - q_k

where Q is the nearest-point quantizer of a finite code book that saturates
to its end points.  Section 2.1 shows E_k = r_{k-1} - r_k, so the errors
telescope: sum_{k<=m} (q_k - x) = -r_m.  Section 2.2 proves |r_k| <= d/2 when
x lies in the hull [c_0, c_N] of the code book (d = largest neighbour gap),
and shows that C = {0, 1}, x = 2 diverges.  For E2M1, d = 2, so |r_k| <= 1 in
normalised units.  The listing zeroes r at the start of every forward and
normalises x = W / s with a block scale fixed for that forward.

Two forms are provided:

* :func:`sigma_delta_exact` -- the recurrence on an arbitrary finite code
  book in exact rational arithmetic (``fractions.Fraction``), with a
  pluggable rounding rule; used for the worked example and the bound tests;
* :func:`sigma_delta_nvfp4` -- the NVFP4 form the hot path computes, in
  binary32: the fixed scale is the NVFP4 recipe of ``oracle.nvfp4`` computed
  once from the fp32 master W; x = clamp(fl(W * rho), -6, 6) (the clamp is
  the "x inside the hull" hypothesis of section 2.2; it only moves values
  that fl rounding pushed a few ulp past 6); v = fl(x + r); q = nearest E2M1
  code; r = v - value(q), which is exact in binary32 and is checked to be.
"""

from __future__ import annotations

from fractions import Fraction
import math
from typing import Callable, List, Sequence, Tuple

import numpy as np

from .formats import e2m1_round, e2m1_decode, e4m3_decode
from .philox import philox4x32
from . import nvfp4

F32 = np.float32


def nearest_saturating(codebook: Sequence[Fraction]) -> Callable[[Fraction], Fraction]:
    """Nearest-point quantizer of a finite sorted code book that saturates to
    the end points (ties go to the lower point; the worked example below
    uses its own rounding rule)."""
    cb = sorted(Fraction(c) for c in codebook)

    def q(v: Fraction) -> Fraction:
        if v <= cb[0]:
            return cb[0]
        if v >= cb[-1]:
            return cb[-1]
        return min(cb, key=lambda c: (abs(v - c), c))
    return q


def sigma_delta_exact(x: Fraction, quantizer: Callable[[Fraction], Fraction],
                      steps: int) -> Tuple[List[Fraction], List[Fraction]]:
    """Run the recurrence from r_0 = 0 for ``steps`` accesses in exact
    arithmetic; returns (q_1..q_R, r_1..r_R)."""
    x = Fraction(x)
    r = Fraction(0)
    qs, rs = [], []
    for _ in range(steps):
        v = x + r
        q = Fraction(quantizer(v))
        r = v - q
        qs.append(q)
        rs.append(r)
    return qs, rs


def normalised_weight(w: np.ndarray, tensor_scale=None, rule: str = "6"):
    """Fixed-scale setup of the NVFP4 chain for an fp32 master ``w`` [R, K]
(block scales by ``rule``, as in :func:`oracle.nvfp4.quantize`):
    returns (x float32 [R, K], scale bytes, s_t, block_zero mask [R, K]).
    ``tensor_scale`` (the s_t of the whole weight) lets a caller run the
    chain on a subset of rows of a larger weight."""
    w = np.asarray(w, dtype=F32)
    R, K = w.shape
    _, sb_bytes, s_t = nvfp4.quantize(w, tensor_scale=tensor_scale, rule=rule)
    s_b = e4m3_decode(sb_bytes).astype(F32)
    s = (s_t * s_b).astype(F32)
    with np.errstate(divide="ignore"):
        rho = (F32(1.0) / s).astype(F32)
    with np.errstate(invalid="ignore"):                      # 0 * inf in zero blocks, replaced below
        x = (w * np.repeat(rho, nvfp4.BLOCK, axis=1)).astype(F32)
    zero = np.repeat(s == 0, nvfp4.BLOCK, axis=1)
    x = np.where(zero, F32(0), x)
    x = np.clip(x, F32(-6.0), F32(6.0)).astype(F32)
    return x, sb_bytes, s_t, zero


def sigma_delta_nvfp4(w: np.ndarray, steps: int, r0: np.ndarray = None, tensor_scale=None,
                      rule: str = "6"):
    """Run ``steps`` Sigma-Delta accesses on the fp32 master ``w`` [R, K].

    Returns a dict with ``codes`` (list of uint8 [R, K] per step, unpacked),
    ``residues`` (list of float32 [R, K] after each step), ``scales``
    (E4M3 bytes [R, K/16]) and ``s_t``.  ``r0`` (float32) continues a chain
    from a saved residue; default zeros.  ``tensor_scale`` as in
    :func:`normalised_weight`; ``rule="4/6"`` fixes the 4/6 block scales of
    the loopquant page's section 2.5 listing (``block_scale_46``).
    """
    x, sb_bytes, s_t, zero = normalised_weight(w, tensor_scale, rule)
    r = np.zeros_like(x) if r0 is None else np.asarray(r0, dtype=F32).copy()
    codes_all, res_all = [], []
    for _ in range(steps):
        v = (x + r).astype(F32)
        codes = e2m1_round(v)
        codes[zero] = 0
        r64 = v.astype(np.float64) - e2m1_decode(codes)
        r_new = r64.astype(F32)
        assert np.array_equal(r_new.astype(np.float64), r64), "residue not exact in fp32"
        r = r_new
        codes_all.append(codes)
        res_all.append(r.copy())
    return {"codes": codes_all, "residues": res_all, "scales": sb_bytes, "s_t": s_t}


def reverse_tail_schedule(w: np.ndarray, n_rtn: int, n_tail: int, tensor_scale=None, rule: str = "6"):
    """Code banks for n_rtn + n_tail accesses with the reverse-order tail
    (loopquant page, section 2.3): the first ``n_rtn`` accesses use the
    plain nearest code; the last ``n_tail`` run a fresh chain from r_0 = 0
    and take its codes in reverse, tail access j using the chain's code
    n_tail - j + 1, so the last access gets the chain's first code (the
    nearest code) and the chain's final residue r_K meets the tail's first
    access.  Returns the list of banks (uint8 [R, K] unpacked), access
    order."""
    chain = sigma_delta_nvfp4(w, n_tail, tensor_scale=tensor_scale, rule=rule)["codes"]
    return [chain[0].copy() for _ in range(n_rtn)] + [c.copy() for c in chain[::-1]]


# --------------------------------------------------- stochastic rounding ----
#: the 15 distinct E2M1 values in increasing order
E2M1_GRID = np.array([-6.0, -4.0, -3.0, -2.0, -1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def sr_round(x: np.ndarray, words: np.ndarray) -> np.ndarray:
    """Stochastic rounding of float32 x in [-6, 6] to E2M1 codes with one
    uint32 random word per element (loopquant page, section 2: a fresh
    random code per access whose expectation is the weight).  With lo the
    largest grid value <= x, hi the next one and u = (word >> 8) / 2^24,
    the code is hi exactly when lo + u (hi - lo) < x (evaluated exactly: in
    float64 both sides are exact), so P(hi) = (x - lo) / (hi - lo) up to
    2^-24; x on the grid (and x = 6) is kept.  A zero value keeps the sign
    bit of x, as the nearest-code quantizer does."""
    x = np.asarray(x, dtype=F32)
    x64 = x.astype(np.float64)
    li = np.searchsorted(E2M1_GRID, x64, side="right") - 1
    li = np.clip(li, 0, E2M1_GRID.size - 1)
    hi_i = np.minimum(li + 1, E2M1_GRID.size - 1)
    lo, hi = E2M1_GRID[li], E2M1_GRID[hi_i]
    u = (np.asarray(words, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) * 2.0 ** -24
    t = lo + u * (hi - lo)                                     # exact
    v = np.where((li < E2M1_GRID.size - 1) & (t < x64), hi, lo)
    mag = np.searchsorted(E2M1_VALUES_POS, np.abs(v)).astype(np.uint8)
    neg = (v < 0) | ((v == 0) & np.signbit(x))
    return mag | (neg.astype(np.uint8) << 3)


E2M1_VALUES_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def sr_words(rows, cols: int, step: int, seed: int, segment: int = 0) -> np.ndarray:
    """Random word of each element of the given rows (row-major index
    e = row * cols + col) at one access: Philox4x32-10 with counter
    (g mod 2^32, g div 2^32, step mod 2^32, segment) for g = e div 4, key
    (seed mod 2^32, seed div 2^32 mod 2^32); element e takes output word
    e mod 4.  Returns uint32 [len(rows), cols]."""
    e = np.asarray(rows, dtype=np.uint64)[:, None] * np.uint64(cols) + np.arange(cols, dtype=np.uint64)[None, :]
    g = e >> np.uint64(2)
    out = philox4x32(g & np.uint64(0xFFFFFFFF), g >> np.uint64(32), int(step) & 0xFFFFFFFF, int(segment),
                     int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    stacked = np.stack(out, axis=-1)                          # [rows, cols, 4]
    return np.take_along_axis(stacked, (e & np.uint64(3)).astype(np.int64)[..., None], axis=-1)[..., 0]


def stochastic_rounding_nvfp4(w: np.ndarray, steps: int, seed: int, step0: int = 0, segment: int = 0,
                              rows=None, tensor_scale=None, rule: str = "6"):
    """Code banks of ``steps`` accesses with stochastic rounding at the same
    fixed NVFP4 scale as the Sigma-Delta chain (x = clamp(W / s, -6, 6));
    access k draws its words at step step0 + k.  ``rows`` selects rows of
    the result (the words still follow the full weight's element indexes).
    Returns a list of uint8 [R, K] unpacked code arrays."""
    x, _, _, zero = normalised_weight(w, tensor_scale, rule)
    R, K = x.shape
    sel = np.arange(R) if rows is None else np.asarray(rows)
    out = []
    for k in range(steps):
        codes = sr_round(x[sel], sr_words(sel, K, step0 + k, seed, segment))
        codes[zero[sel]] = 0
        out.append(codes)
    return out


# ------------------------------------------------------------------ F4b ----

def two_point_code(x: float, k: int) -> int:
    """Access k (k >= 1) of the stateless two-point chain (F4b) for one
    normalised float32 value x in [-6, 6], in exact rationals.

    The loopquant page names F4b, the "two-point closed-form difference"
    used in its code-generation microbenchmark, but gives no formula; the
    reading taken (recorded in the design notes): with lo the largest E2M1
    value <= x, hi the next one and p = (x - lo) / (hi - lo), access k takes
    hi exactly when floor(k p) - floor((k - 1) p) = 1, else lo, so after m
    accesses the code sum is m lo + (hi - lo) floor(m p).  Values on the
    grid (and 6) are kept; a zero value keeps the sign bit of x."""
    fx = Fraction(float(np.float32(x)))
    vals = [Fraction(v).limit_denominator(2) for v in E2M1_GRID]
    li = max(i for i, v in enumerate(vals) if v <= fx)
    if li == len(vals) - 1 or vals[li] == fx:
        v = vals[li]
    else:
        lo, hi = vals[li], vals[li + 1]
        p = (fx - lo) / (hi - lo)
        up = math.floor(k * p) - math.floor((k - 1) * p)
        v = hi if up == 1 else lo
    mag = int(np.searchsorted(E2M1_VALUES_POS, abs(float(v))))
    neg = v < 0 or (v == 0 and np.signbit(np.float32(x)))
    return mag | (8 if neg else 0)


def two_point_nvfp4(w: np.ndarray, accesses, rows=None, tensor_scale=None, rule: str = "6"):
    """F4b codes of the given accesses (1-based indexes k) at the fixed
    NVFP4 scale of the Sigma-Delta chain; ``rows`` selects rows.  Returns a
    dict k -> uint8 [R, K] unpacked codes.  Pure-Python rationals: small
    inputs only."""
    x, _, _, zero = normalised_weight(w, tensor_scale, rule)
    sel = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    out = {}
    for k in accesses:
        codes = np.array([[two_point_code(v, k) for v in x[r]] for r in sel], np.uint8)
        codes[zero[sel]] = 0
        out[k] = codes
    return out
