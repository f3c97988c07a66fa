"""Pins for the oracle's Sigma-Delta recurrence and its GEMMs (CPU only)."""
import os
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import formats as F, nvfp4, mxfp4, sigma_delta as SD, gemm
from block_scaled_fp4_mxfp4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden_rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append([Fraction(t) for t in line.split()])
    return out


def test_worked_example_x03_integer_grid():
    # loopquant page, section 2.1: x = 0.3, integer grid, floor(v + 1/2)
    q_int = lambda v: Fraction(math.floor(v + Fraction(1, 2)))
    qs, rs = SD.sigma_delta_exact(Fraction(3, 10), q_int, 8)
    rows = _golden_rows("sigma_delta_x03.txt")
    x = Fraction(3, 10)
    prefix = Fraction(0)
    for k, (row, q, r) in enumerate(zip(rows, qs, rs), start=1):
        kk, v, qq, rr, pe = row
        assert kk == k and q == qq and r == rr
        prefix += q - x
        assert prefix == pe == -r                 # prefix error = -r_k
        assert abs(r) <= Fraction(1, 2)
    # static RTN: 0 every step, error -0.3 each step, diverging linearly
    assert all(q_int(x) == 0 for _ in range(8))


def test_telescoping_and_bound_on_random_code_books():
    rng = np.random.default_rng(40)
    for trial in range(60):
        n = int(rng.integers(2, 9))
        cb = sorted(set(Fraction(int(v), int(rng.integers(1, 5)))
                        for v in rng.integers(-20, 20, size=n)))
        if len(cb) < 2:
            continue
        d = max(b - a for a, b in zip(cb, cb[1:]))
        x = cb[0] + (cb[-1] - cb[0]) * Fraction(int(rng.integers(0, 1000)), 999)
        qs, rs = SD.sigma_delta_exact(x, SD.nearest_saturating(cb), 50)
        s = Fraction(0)
        for m, (q, r) in enumerate(zip(qs, rs), start=1):
            s += q - x
            assert s == -r                       # section 2.1 telescoping
            assert abs(r) <= d / 2               # section 2.2 bound
            assert abs(s / m) <= d / (2 * m)     # mean error <= d / (2m)


def test_divergence_outside_hull():
    # section 2.2: C = {0, 1}, x = 2 -> residue grows without bound
    qs, rs = SD.sigma_delta_exact(Fraction(2), SD.nearest_saturating([0, 1]), 10)
    assert rs == [Fraction(k) for k in range(1, 11)]


def test_e2m1_code_book_bound_is_one():
    cb = sorted(set(Fraction(float(v)) for v in F.E2M1_VALUES))
    rng = np.random.default_rng(41)
    for _ in range(40):
        x = Fraction(int(rng.integers(-6000, 6001)), 1000)
        _, rs = SD.sigma_delta_exact(x, SD.nearest_saturating(cb), 32)
        assert max(abs(r) for r in rs) <= 1


def test_nvfp4_chain_step1_is_rtn_and_bound_holds():
    w = synth.normal_f32(42, (48, 256), 0.02)
    w[3, 16:32] = 0.0                                        # a zero block
    out = SD.sigma_delta_nvfp4(w, 32)
    codes_rtn, sb, st = nvfp4.quantize(w)
    # loopquant page, section 2.3: the first code of the chain is the RTN code
    assert np.array_equal(out["codes"][0], codes_rtn)
    assert np.array_equal(out["scales"], sb) and out["s_t"] == st
    for r in out["residues"]:
        assert np.abs(r).max() <= 1.0                        # |r_k| <= d/2 = 1
    assert not any(c[3, 16:32].any() for c in out["codes"])


def test_nvfp4_chain_telescopes_within_fp32_rounding():
    w = synth.normal_f32(43, (16, 128), 0.02)
    out = SD.sigma_delta_nvfp4(w, 32)
    x, _, _, _ = SD.normalised_weight(w)
    x = x.astype(np.float64)
    acc = np.zeros_like(x)
    for m, (c, r) in enumerate(zip(out["codes"], out["residues"]), start=1):
        acc += F.e2m1_decode(c) - x
        # each v = fl(x + r) rounds by at most half an ulp of 8 (2**-21)
        assert np.abs(acc + r.astype(np.float64)).max() <= m * 2.0 ** -21
        assert np.abs(acc / m).max() <= 1.0 / m + 2.0 ** -21


def test_nvfp4_chain_resume_is_exact():
    w = synth.normal_f32(44, (8, 64), 0.02)
    full = SD.sigma_delta_nvfp4(w, 12)
    a = SD.sigma_delta_nvfp4(w, 5)
    b = SD.sigma_delta_nvfp4(w, 7, r0=a["residues"][-1])
    for k in range(7):
        assert np.array_equal(full["codes"][5 + k], b["codes"][k])
        assert np.array_equal(full["residues"][5 + k], b["residues"][k])


# ------------------------------------------------------------------ GEMM --

def test_gemm_one_hot_rows_return_weight_rows():
    w = synth.normal_f32(45, (24, 64), 0.02)
    bc, bs, bst = nvfp4.quantize(w)
    a = np.zeros((3, 64), F32)
    a[0, 5] = 1.0; a[1, 63] = 1.0; a[2, 0] = -1.0
    ac, as_, ast = nvfp4.quantize(a)
    y = gemm.w4a4_nvfp4(ac, as_, ast, bc, bs, bst)
    wd = nvfp4.dequantize(bc, bs, bst)
    ad = nvfp4.dequantize(ac, as_, ast)
    # a one-hot row dequantizes to a single non-zero (6 * s_b * s_t, not
    # exactly 1 because s_t = 1/1536 rounds in fp32)
    assert np.count_nonzero(ad[0]) == 1 and abs(ad[0, 5] - 1) < 1e-6
    assert np.array_equal(y[0], ad[0, 5] * wd[:, 5]) and np.array_equal(y[1], ad[1, 63] * wd[:, 63])
    assert np.array_equal(y[2], ad[2, 0] * wd[:, 0])


def test_gemm_matches_exact_rational_brute_force():
    x = synth.heavy_tailed_f32(46, 47, (4, 64))
    w = synth.normal_f32(48, (5, 64), 0.02)
    ac, as_, ast = nvfp4.quantize(x)
    bc, bs, bst = nvfp4.quantize(w)
    y = gemm.w4a4_nvfp4(ac, as_, ast, bc, bs, bst)
    A = nvfp4.dequantize(ac, as_, ast)
    B = nvfp4.dequantize(bc, bs, bst)
    for i in range(4):
        for j in range(5):
            ex = sum(Fraction(float(A[i, k])) * Fraction(float(B[j, k])) for k in range(64))
            assert abs(Fraction(float(y[i, j])) - ex) <= sum(abs(Fraction(float(A[i, k])) * Fraction(float(B[j, k]))) for k in range(64)) * Fraction(64, 2 ** 53) + Fraction(1, 2 ** 200)
    # MXFP4 and W4A16 variants on the same data
    mc, ms = mxfp4.quantize(x); wc, ws = mxfp4.quantize(w)
    ym = gemm.w4a4_mxfp4(mc, ms, wc, ws)
    assert np.allclose(ym, mxfp4.dequantize(mc, ms) @ mxfp4.dequantize(wc, ws).T, rtol=0, atol=0)
    xb = synth.f32_to_bf16_bits(x)
    yh = gemm.w4a16(xb, bc, bs, bst)
    assert np.allclose(yh, F.bf16_bits_to_f32(xb).astype(np.float64) @ B.T, rtol=0, atol=0)


def test_rel_err_metric():
    y = np.array([[1.0, 0.0], [0.0, 2.0]])
    whole, row, mx = gemm.rel_err(y * (1 + 1e-4), y)
    assert abs(whole - 1e-4) < 1e-12 and abs(row - 1e-4) < 1e-12 and abs(mx - 1e-4) < 1e-12


def test_sigma_delta_on_46_scales_keeps_the_residue_bound():
    # the section 2.2 bound |r_k| <= d/2 = 1 holds for either 4/6 candidate,
    # since both keep |x| <= 6 (the page's argument); the chain also averages
    # back to x
    w = synth.normal_f32(307, (16, 256), 0.02)
    ref = SD.sigma_delta_nvfp4(w, 32, rule="4/6")
    assert max(np.abs(r).max() for r in ref["residues"]) <= 1.0
    x, _, _, _ = SD.normalised_weight(w, rule="4/6")
    mean_q = np.mean([F.e2m1_decode(c) for c in ref["codes"]], axis=0)
    assert np.abs(mean_q - x).max() <= 1.0 / 32 + 1e-6


def test_reverse_tail_schedule():
    # loopquant page, section 2.3: B plain nearest-code accesses, then a fresh
    # chain of K codes used in reverse; the last access takes the nearest
    # code and the tail's total error is the chain's -r_K, now met at the
    # tail's first access
    w = synth.normal_f32(44, (24, 128), 0.02)
    w[2, :16] = 0.0
    B, K = 3, 6
    banks = SD.reverse_tail_schedule(w, B, K)
    assert len(banks) == B + K
    codes_rtn, _, _ = nvfp4.quantize(w)
    for b in banks[:B]:
        assert np.array_equal(b, codes_rtn)
    assert np.array_equal(banks[-1], codes_rtn)              # last access: the chain's first code
    chain = SD.sigma_delta_nvfp4(w, K)
    assert np.array_equal(banks[B], chain["codes"][K - 1])   # tail entrance: the chain's last code
    x, _, _, _ = SD.normalised_weight(w)
    x = x.astype(np.float64)
    tail_err = sum(F.e2m1_decode(c) - x for c in banks[B:])
    assert np.abs(tail_err + chain["residues"][K - 1].astype(np.float64)).max() <= K * 2.0 ** -21
    # K = 1: every access is the nearest code
    assert all(np.array_equal(b, codes_rtn) for b in SD.reverse_tail_schedule(w, 2, 1))
    # the worked example of section 2.1 reversed: x = 0.3 on the integer grid
    q_int = lambda v: Fraction(math.floor(v + Fraction(1, 2)))
    qs, _ = SD.sigma_delta_exact(Fraction(3, 10), q_int, 8)
    assert [int(q) for q in qs[::-1]] == [0, 0, 0, 1, 0, 0, 1, 0]


# ------------------------------------------------- stochastic rounding ----

def test_philox_known_answer_vectors():
    from oracle.philox import philox4x32
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    n = 0
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            v = [int(t, 16) for t in line.split()]
            got = [int(a) for a in philox4x32(*v[:4], v[4], v[5])]
            assert got == v[6:], line
            n += 1
    assert n == 3


def test_sr_decision_boundaries():
    # x = 0.6 between 0.5 and 1: P(hi) = 0.2, hi exactly when u < 0.2
    b = int(0.2 * 2 ** 24)                        # 3355443.2 -> u = 3355443 / 2^24 < 0.2
    words = np.array([b << 8, (b + 1) << 8, 0, 0xFFFFFFFF], np.uint32)
    x = np.full(4, 0.6, np.float32)
    got = F.e2m1_decode(SD.sr_round(x, words))
    assert list(got) == [1.0, 0.5, 1.0, 0.5]
    # exactly at the threshold (t == x) the lower value is kept
    x = np.array([0.75], np.float32)              # p = 0.5
    assert F.e2m1_decode(SD.sr_round(x, np.array([(1 << 23) << 8], np.uint32)))[0] == 0.5
    assert F.e2m1_decode(SD.sr_round(x, np.array([((1 << 23) - 1) << 8], np.uint32)))[0] == 1.0
    # grid points, the ends and signed zeros are kept whatever the word
    grid = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    for word in (0, 0x12345678, 0xFFFFFFFF):
        c = SD.sr_round(grid, np.full(grid.size, word, np.uint32))
        np.testing.assert_array_equal(F.e2m1_decode(c), grid)
    assert SD.sr_round(np.array([-0.0], np.float32), np.array([0], np.uint32))[0] == 0x8
    assert SD.sr_round(np.array([-0.2], np.float32), np.array([0], np.uint32))[0] == 0x8            # -0.2 up to -0
    assert SD.sr_round(np.array([-0.2], np.float32), np.array([0xFFFFFFFF], np.uint32))[0] == 0x9   # or down to -0.5


def test_sr_is_unbiased_and_brackets_x():
    rng = np.random.default_rng(45)
    x = rng.uniform(-6, 6, 64).astype(np.float32)
    n = 4096
    vals = np.stack([F.e2m1_decode(SD.sr_round(x, SD.sr_words([0], 64, k, 7)[0])) for k in range(n)])
    lo = SD.E2M1_GRID[np.searchsorted(SD.E2M1_GRID, x.astype(np.float64), side="right") - 1]
    assert np.all((vals == lo) | (vals > lo))
    assert np.all(vals <= lo + 2.0)
    gap = np.diff(SD.E2M1_GRID).max()
    # |mean - x| within 6 standard errors (sd <= gap / 2)
    assert np.all(np.abs(vals.mean(axis=0) - x) <= 6 * (gap / 2) / np.sqrt(n))


def test_sr_words_counter_layout():
    # four consecutive elements share one Philox call (output words 0..3);
    # steps, segments and seeds give different streams; a row's words do not
    # depend on which other rows are drawn
    from oracle.philox import philox4x32
    w = SD.sr_words([0, 1], 8, 3, 0x1_0000_0002, segment=5)
    ref = philox4x32(np.arange(4), 0, 3, 5, 2, 1)
    np.testing.assert_array_equal(w.reshape(-1), np.stack(ref, axis=-1).reshape(-1))
    assert not np.array_equal(SD.sr_words([0], 64, 0, 7), SD.sr_words([0], 64, 1, 7))
    assert not np.array_equal(SD.sr_words([0], 64, 0, 7, 1), SD.sr_words([0], 64, 0, 7, 0))
    np.testing.assert_array_equal(SD.sr_words([3, 9], 16, 2, 11)[1], SD.sr_words([9], 16, 2, 11)[0])
    ws = synth.normal_f32(46, (12, 64), 0.02)
    full = SD.stochastic_rounding_nvfp4(ws, 2, seed=9)
    part = SD.stochastic_rounding_nvfp4(ws, 2, seed=9, rows=[4, 11])
    np.testing.assert_array_equal(full[1][[4, 11]], part[1])


# ----------------------------------------------------------------- F4b ----

def test_two_point_chain_pins():
    # p = 1/2 alternates lo, hi; grid points and the ends are kept
    assert [SD.two_point_code(0.75, k) for k in range(1, 7)] == [0x1, 0x2] * 3
    for x in (0.0, 0.5, 1.5, 4.0, 6.0, -6.0, -3.0):
        want = F.e2m1_round(np.array([x], np.float32))[0]
        assert all(SD.two_point_code(x, k) == want for k in (1, 2, 5, 100))
    # x = 0.3 on [0, 0.5] is p = 0.6: floor(0.6 k) - floor(0.6 (k - 1))
    assert [SD.two_point_code(0.3, k) & 7 for k in range(1, 6)] == [0, 1, 0, 1, 1]
    # negative side, hi = -0: x = -0.125 in [-0.5, 0], p = 0.75
    assert [SD.two_point_code(-0.125, k) for k in range(1, 6)] == [0x9, 0x8, 0x8, 0x8, 0x9]
    # the section 2.1 worked example's p = 0.3 on the integer grid, in the same
    # closed form, gives 0,0,0,1,0,0,1,0
    seq = [math.floor(Fraction(3, 10) * k) - math.floor(Fraction(3, 10) * (k - 1)) for k in range(1, 9)]
    assert seq == [0, 0, 0, 1, 0, 0, 1, 0]


def test_two_point_chain_sum_and_brackets():
    # after m accesses the code sum is m lo + (hi - lo) floor(m p): the prefix
    # error lies in (-(hi - lo), 0]; every code is lo or hi
    rng = np.random.default_rng(47)
    xs = rng.uniform(-6, 6, 40).astype(np.float32)
    for x in xs:
        fx = Fraction(float(x))
        vals = [Fraction(v).limit_denominator(2) for v in SD.E2M1_GRID]
        li = max(i for i, v in enumerate(vals) if v <= fx)
        lo = vals[li]
        hi = vals[min(li + 1, len(vals) - 1)]
        tot = Fraction(0)
        for m in range(1, 65):
            v = Fraction(float(F.e2m1_decode(np.array([SD.two_point_code(x, m)]))[0]))
            assert v in (lo, hi)
            tot += v - fx
            assert -(hi - lo) < tot <= 0 or (hi == lo and tot == 0)
    # tiny values next to zero are exact too: x = -2^-140 gives
    # p = 1 - 2^-139, so access 1 takes lo and the next ones hi (-0)
    tiny = np.float32(-2.0 ** -140)
    assert [SD.two_point_code(tiny, k) for k in (1, 2, 3, 1000)] == [0x9, 0x8, 0x8, 0x8]
    assert [SD.two_point_code(-tiny, k) for k in (1, 2, 1000)] == [0x0, 0x0, 0x0]
