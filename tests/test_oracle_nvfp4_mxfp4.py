"""Pins for the oracle's NVFP4 / MXFP4 quantizers, the block-32 Hadamard
transform and the balance scale (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import formats as F, nvfp4, mxfp4, balance
from block_scaled_fp4_mxfp4_amd import synth

F32 = np.float32


# ------------------------------------------------------------------ NVFP4 --

def test_nvfp4_tensor_scale_is_amax_over_1536():
    # loopquant page section 2.2: s_tensor = max|W| / (6 * 256)
    x = synth.normal_f32(11, (8, 64), 3.0)
    _, _, st = nvfp4.quantize(x)
    a = np.abs(x).max()
    assert st == F32(a / F32(1536))
    assert abs(float(st) * 1536 / float(a) - 1) < 2 ** -23


def test_nvfp4_block_scale_is_smallest_e4m3_at_least_amax_over_6st():
    x = synth.heavy_tailed_f32(12, 13, (32, 256))
    codes, sb, st = nvfp4.quantize(x)
    table = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    a_b = np.abs(x).reshape(32, 16, 16).max(-1)
    for i in range(32):
        for j in range(16):
            y = float(F32(a_b[i, j] / F32(F32(6) * st)))
            want = np.nonzero(table >= y)[0][0]
            assert sb[i, j] == want


def test_nvfp4_codes_are_nearest_to_normalised_value():
    x = synth.heavy_tailed_f32(14, 15, (16, 128))
    codes, sb, st = nvfp4.quantize(x)
    s = (st * F.e4m3_decode(sb).astype(F32)).astype(F32)
    rho = (F32(1) / s).astype(F32)
    mags = [Fraction(m) for m in (0, .5, 1, 1.5, 2, 3, 4, 6)]
    exact_mismatch = 0
    for i in range(16):
        for k in range(128):
            v = Fraction(float(F32(x[i, k] * rho[i, k // 16])))
            want = min(range(8), key=lambda m: (abs(abs(v) - mags[m]), m & 1))
            assert codes[i, k] & 7 == want
            # against the exact quotient x / s (no reciprocal rounding)
            vq = Fraction(float(x[i, k])) / Fraction(float(s[i, k // 16]))
            wq = min(range(8), key=lambda m: (abs(abs(vq) - mags[m]), m & 1))
            exact_mismatch += int(wq != want)
    assert exact_mismatch == 0


def test_nvfp4_normalised_magnitude_bounded_by_6():
    # loopquant page section 2.2: the rounded-up E4M3 block scale keeps |x/s| <= 6
    x = synth.heavy_tailed_f32(16, 17, (64, 512))
    codes, sb, st = nvfp4.quantize(x)
    s = st * F.e4m3_decode(sb)
    v = np.abs(x.astype(np.float64)) / np.repeat(s, 16, axis=1)
    assert v.max() <= 6 * (1 + 2 ** -21)


def test_nvfp4_block_max_maps_to_six_when_scale_is_normal():
    # ceil to E4M3 loses at most one part in 8 for normal E4M3 scales, so the
    # block maximum lands in (5.33, 6] -> code magnitude 6
    x = synth.heavy_tailed_f32(18, 19, (64, 512))
    codes, sb, st = nvfp4.quantize(x)
    blocks = np.abs(x).reshape(64, 32, 16)
    cb = codes.reshape(64, 32, 16)
    normal = F.e4m3_decode(sb) >= 2 ** -6
    arg = blocks.argmax(-1)
    top = np.take_along_axis(cb, arg[..., None], -1)[..., 0] & 7
    assert np.all(top[normal] == 7)


def test_nvfp4_block_max_over_rms_at_most_4():
    # GDN page, background box "NVFP4 and W4A4": block max/RMS <= 4 in a
    # 16-element block (= sqrt(16)); equality iff one non-zero element
    x = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(20, 21, (256, 1024)))
    x = F.bf16_bits_to_f32(x).astype(np.float64).reshape(256, -1, 16)
    r = np.abs(x).max(-1) / np.sqrt((x * x).mean(-1))
    assert r.max() <= 4 + 1e-12
    one = np.zeros((1, 16)); one[0, 5] = 3.0
    assert np.abs(one).max() / np.sqrt((one ** 2).mean()) == 4.0


def test_nvfp4_storage_is_4_5_bits():
    # MACaQ page, image-diffusion comparison: NVFP4 costs 4.50 bits/element
    x = synth.normal_f32(22, (4, 256))
    codes, sb, _ = nvfp4.quantize(x)
    packed = F.pack_nibbles(codes)
    assert (packed.nbytes + sb.nbytes) * 8 / x.size == 4.5


def test_nvfp4_exactly_representable_tensor_round_trips():
    grid = np.array([6, 4, 3, 2, 1.5, 1, .5, 0, -.5, -1, -1.5, -2, -3, -4, -6, 0], F32)
    for k in (-20, -3, 0, 5, 30):
        x = np.tile(grid * F32(2.0 ** k), (3, 4)).astype(F32)
        codes, sb, st = nvfp4.quantize(x)
        assert np.array_equal(nvfp4.dequantize(codes, sb, st), x.astype(np.float64))
        assert np.all(F.e4m3_decode(sb) == 256.0)


def test_nvfp4_zero_tensor_and_given_scale():
    z = np.zeros((2, 32), F32)
    codes, sb, st = nvfp4.quantize(z)
    assert st == 0 and not codes.any() and not sb.any()
    x = synth.normal_f32(23, (2, 32))
    c1, s1, st1 = nvfp4.quantize(x)
    c2, s2, st2 = nvfp4.quantize(x, tensor_scale=st1)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and st1 == st2
    c3, s3, st3 = nvfp4.quantize(x, tensor_scale=F32(0))
    assert not c3.any() and not s3.any()


def test_nvfp4_error_in_plausible_range():
    # sanity only: the GDN page reports A4 errors of 7.5-9.2 % on real data
    x = synth.heavy_tailed_f32(24, 25, (256, 1024))
    codes, sb, st = nvfp4.quantize(x)
    d = nvfp4.dequantize(codes, sb, st) - x
    e = np.linalg.norm(d) / np.linalg.norm(x)
    assert 0.04 < e < 0.15


# ------------------------------------------------------------- Hadamard --

def test_sylvester_hadamard_is_orthogonal():
    H = scipy.linalg.hadamard(32)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=H.dtype))
    assert set(np.unique(H)) == {-1, 1}


def test_fwht_matches_dense_sylvester_exactly_on_integers():
    H = scipy.linalg.hadamard(32).astype(np.float64)
    rng = np.random.default_rng(5)
    z = rng.integers(-1000, 1000, size=(20, 96)).astype(F32)
    y = mxfp4.fwht32_stages(z).astype(np.float64)
    ref = (z.astype(np.float64).reshape(20, 3, 32) @ H.T).reshape(20, 96)
    assert np.array_equal(y, ref)


def test_fwht_matches_dense_on_floats():
    H = scipy.linalg.hadamard(32).astype(np.float64) / np.sqrt(32)
    x = synth.heavy_tailed_f32(26, 27, (16, 256))
    y = mxfp4.hadamard32_scale(x).astype(np.float64)
    ref = (x.astype(np.float64).reshape(16, 8, 32) @ H.T).reshape(16, 256)
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()
    # orthonormal and symmetric -> applying it twice is the identity
    yy = mxfp4.hadamard32_scale(mxfp4.hadamard32_scale(x)).astype(np.float64)
    assert np.abs(yy - x).max() <= 1e-5 * np.abs(x).max()


def test_scale_then_rotate_leaves_product_unchanged():
    # MACaQ page, core method (ii): X' D B (W D^-1 B)^T = X W^T
    x = synth.heavy_tailed_f32(28, 29, (32, 256))
    w = synth.normal_f32(30, (48, 256), 0.02)
    t64, t32, u32 = balance.balance_scale(w, x)
    xp = mxfp4.hadamard32_scale(x, t32).astype(np.float64)
    wp = mxfp4.hadamard32_scale(w, u32).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    got = xp @ wp.T
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-5


# ---------------------------------------------------------------- MXFP4 --

def test_mxfp4_scale_is_power_of_two_with_block_max_in_4_8():
    y = synth.heavy_tailed_f32(31, 32, (32, 512))
    codes, sc = mxfp4.quantize(y)
    a_b = np.abs(y.astype(np.float64)).reshape(32, 16, 32).max(-1)
    s = F.e8m0_decode(sc)
    ratio = a_b / s
    assert np.all((ratio >= 4) & (ratio < 8))
    tt = torch.from_numpy(sc.copy()).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(tt, s)


def test_mxfp4_codes_nearest_and_saturate():
    y = synth.heavy_tailed_f32(33, 34, (8, 128))
    codes, sc = mxfp4.quantize(y)
    mags = [Fraction(m) for m in (0, .5, 1, 1.5, 2, 3, 4, 6)]
    for i in range(8):
        for k in range(128):
            v = Fraction(float(y[i, k])) / (Fraction(2) ** (int(sc[i, k // 32]) - 127))
            want = min(range(8), key=lambda m: (abs(abs(v) - mags[m]), m & 1))
            assert codes[i, k] & 7 == want


def test_mxfp4_storage_is_4_25_bits_and_zero_block():
    # MACaQ page, MXFP4 box: about 4.25 bits per element
    y = synth.normal_f32(35, (4, 256))
    y[1, 32:64] = 0
    codes, sc = mxfp4.quantize(y)
    assert (F.pack_nibbles(codes).nbytes + sc.nbytes) * 8 / y.size == 4.25
    assert sc[1, 1] == 0 and not codes[1, 32:64].any()


def test_mxfp4_subnormal_and_extreme_blocks():
    y = np.zeros((1, 96), F32)
    y[0, 0] = np.float32(1e-45)                  # smallest subnormal
    y[0, 32] = np.float32(3e38)                  # near the fp32 max
    y[0, 64:96] = F32(6.0)
    codes, sc = mxfp4.quantize(y)
    assert sc[0, 0] == 0                         # exponent clamped at -127
    assert sc[0, 1] == 127 + 127 - 2             # floor(log2 3e38) = 127
    # a block of 6.0: floor(log2 6) = 2 -> e = 0 -> v = 6 -> magnitude index 7
    assert sc[0, 2] == 127 and np.all(codes[0, 64:96] == 0x7)
    assert mxfp4.dequantize(codes, sc)[0, 0] == 0.0


def test_balance_scale_closed_form():
    rng = np.random.default_rng(36)
    w = rng.standard_normal((50, 4)) * np.array([1.0, 2.0, 0.5, 4.0])
    x = rng.standard_normal((70, 4)) * np.array([3.0, 1.0, 10.0, 0.25])
    t64, t32, u32 = balance.balance_scale(w, x)
    sig = np.sqrt(((w - w.mean(0)) ** 2).mean(0))
    rms = np.sqrt((x ** 2).mean(0))
    assert np.allclose(t64, sig ** 0.75 / rms ** 0.25, rtol=1e-14)
    assert t32.dtype == np.float32 and u32.dtype == np.float32
    assert np.allclose(t32.astype(np.float64) * u32, 1, rtol=2e-7)


# Hand-worked values of the balance scale ("MACaQ", core method step (i):
# t = sigma_W^0.75 / rms_x^0.25, range-clipped).  Each column below is built
# so that sigma (population std over the weight rows) and rms are exact
# powers of two, zero, or fixed values; the expected t is written out here,
# not recomputed with the oracle's formula.
def _balance_columns():
    # W: 4 rows; X: 4 rows.  Column j: (W column, X column, expected t)
    cols = [
        ([16, -16, 16, -16], [16, 16, -16, 16], 4.0),            # 16^0.75 / 16^0.25 = 8 / 2
        ([256, -256, 256, -256], [1, -1, 1, 1], 64.0),           # 256^0.75 / 1 = 2^6
        ([1, -1, -1, 1], [256, 256, 256, -256], 0.25),           # 1 / 256^0.25 = 2^-2
        ([5, 5, 5, 5], [1, 1, -1, 1], 2.0 ** -16),               # sigma = 0 -> 1e-12: t = 1e-9, clipped up
        ([1024, -1024, 1024, -1024], [0, 0, 0, 0], 2.0 ** 16),   # rms = 0 -> 1e-12: t = 181019, clipped down
        ([1, -1, 1, -1], [0, 0, 0, 0], 1000.0),                  # rms floor 1e-12 -> 1 / (1e-12)^0.25 = 1000
        ([2, -2, 2, -2], [16, -16, 16, -16], 2.0 ** -0.25),      # 2^(0.75 - 1)
        ([3, 3, -1, -1], [2, 2, 2, 2], 2.0 ** 0.5),             # sigma 2 (mean 1), rms 2: 2^(0.75 - 0.25)
    ]
    w = np.array([c[0] for c in cols], dtype=np.float64).T.copy()
    x = np.array([c[1] for c in cols], dtype=np.float64).T.copy()
    return w, x, np.array([c[2] for c in cols])


def test_balance_scale_hand_worked_values():
    w, x, want = _balance_columns()
    t64, t32, u32 = balance.balance_scale(w, x)
    exact = [0, 1, 2, 3, 4]                  # powers of two: no rounding anywhere
    assert np.array_equal(t64[exact], want[exact])
    assert np.array_equal(t32[exact], want[exact].astype(np.float32))
    assert np.array_equal(u32[exact], (1.0 / want[exact]).astype(np.float32))
    # the rest are one or two fp64 roundings away from the written-out value
    assert np.allclose(t64, want, rtol=4e-16, atol=0)


def test_balance_scale_orientation_and_population_std():
    # alpha belongs to sigma_W: swapping the exponents would give
    # 16^0.25 / 256^0.75 = 2^-4 for this column instead of 2^4
    w = np.array([[16.0], [-16.0]])
    x = np.array([[256.0], [256.0]])
    t64, _, _ = balance.balance_scale(w, x)
    assert t64[0] == 2.0 ** 3 / 2.0 ** 2
    # population std (ddof = 0): +-2 over 4 rows is exactly 2 (the sample std
    # would be 2 sqrt(4/3))
    w = np.array([[2.0], [-2.0], [2.0], [-2.0]])
    x = np.ones((4, 1))
    t64, _, _ = balance.balance_scale(w, x)
    assert t64[0] == 2.0 ** 0.75


# ------------------------------------------------ NVFP4, 4/6 block scales ----
# loopquant page, section 2.2 (the 4/6 block scaling keeps |x/s| <= 6 with
# the block maximum mapped to 6 or to 4) and the section 2.5 listing
# (block_scale_46).  The choice between the two candidates is by block
# squared error (reading adopted; ties to 6).

def _e4m3_ceil_brute(y):
    vals = F.E4M3_VALUES[:127].astype(np.float64)
    if y <= 0:
        return 0
    ok = np.nonzero(vals >= y)[0]
    return int(ok[0]) if ok.size else 126


def test_nvfp46_exactly_representable_blocks_pick_the_exact_candidate():
    st = np.float32(0.0625)          # candidate scales: max 4 -> 16 x st = 1, max 6 -> 16 x st = 1
    four = [4, 2, 1, 0.5, 1.5, 3, 0, -4, -2, -1, -0.5, -1.5, -3, 0, 4, 2]      # exact at s = 1 only with max -> 4
    six = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0]      # exact at s = 1 only with max -> 6
    x = np.array([four + six + [0.0] * 16], np.float32)
    codes, scales, s_t = nvfp4.quantize(x, tensor_scale=st, rule="4/6")
    assert s_t == st
    assert list(scales[0]) == [0x58, 0x58, 0x00]          # E4M3 0x58 = 16; zero block: 0 (tie -> 6)
    np.testing.assert_array_equal(F.e2m1_decode(codes[0, :32]), np.array(four + six, np.float64))
    # the max -> 6 rule alone cannot represent the first block
    c6, s6, _ = nvfp4.quantize(x, tensor_scale=st)
    assert s6[0, 0] != 0x58 and not np.array_equal(F.e2m1_decode(c6[0, :16]), np.array(four, np.float64))


def test_nvfp46_choice_follows_the_exact_block_error():
    x = synth.heavy_tailed_f32(301, 302, (64, 256))
    st = nvfp4.tensor_scale_from_amax(np.abs(x).max())
    codes, scales, _ = nvfp4.quantize(x, rule="4/6")
    xb = x.reshape(64, 16, 16).astype(np.float64)
    picked4 = decided = 0
    for r in range(64):
        for b in range(16):
            blk = xb[r, b]
            a = np.abs(blk).max()
            errs, bytes_ = {}, {}
            for target in (6, 4):
                y = np.float32(np.float32(a) / np.float32(np.float32(target) * st))
                sb = _e4m3_ceil_brute(float(y))
                s = np.float64(np.float32(st * np.float32(F.E4M3_VALUES[sb])))
                v = (blk / s) if s > 0 else np.zeros(16)
                q = np.array([F.E2M1_VALUES[np.argmin(np.abs(F.E2M1_VALUES - vi))] * 1.0 for vi in v])
                errs[target] = float(np.sum((blk - s * q) ** 2))
                bytes_[target] = sb
            assert scales[r, b] in (bytes_[6], bytes_[4])
            e6, e4 = errs[6], errs[4]
            if abs(e6 - e4) > 1e-5 * max(e6, e4, 1e-30):
                decided += 1
                want = bytes_[4] if e4 < e6 else bytes_[6]
                assert scales[r, b] == want, (r, b, e4, e6)
                picked4 += want == bytes_[4] and bytes_[4] != bytes_[6]
    assert decided > 900 and picked4 > 50                    # both candidates occur


def test_nvfp46_normalised_magnitude_and_block_max_at_4():
    x = synth.heavy_tailed_f32(303, 304, (32, 512))
    codes, scales, st = nvfp4.quantize(x, rule="4/6")
    s = (np.float32(st) * F.e4m3_decode(scales).astype(np.float32)).astype(np.float32)
    rho = (np.float32(1.0) / s).astype(np.float32)
    v = (x * np.repeat(rho, 16, axis=1)).astype(np.float32)
    assert np.abs(v).max() <= 6.0 * (1 + 2.0 ** -20)
    # a block that took the max -> 4 candidate with a normal scale has its
    # maximum on code value 4
    c6, s6, _ = nvfp4.quantize(x)
    took4 = (scales != s6) & (scales >= 0x08)                  # normal E4M3 scale bytes
    vals = np.abs(F.e2m1_decode(codes)).reshape(32, 32, 16)
    xa = np.abs(x).reshape(32, 32, 16)
    imax = xa.argmax(axis=-1)
    vmax = np.take_along_axis(vals, imax[..., None], axis=-1)[..., 0]
    assert took4.sum() > 20
    np.testing.assert_array_equal(vmax[took4], 4.0)


def test_nvfp46_total_error_not_above_max_to_6():
    x = synth.heavy_tailed_f32(305, 306, (16, 1024))
    c6, s6, st = nvfp4.quantize(x)
    c46, s46, _ = nvfp4.quantize(x, rule="4/6")
    e6 = np.sum((nvfp4.dequantize(c6, s6, st) - x) ** 2)
    e46 = np.sum((nvfp4.dequantize(c46, s46, st) - x) ** 2)
    assert e46 <= e6 * (1 + 1e-6) and e46 < 0.99 * e6


# ------------------------------------- fused-projection scale harmonization ----
# "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
# Recurrent Half of a Hybrid 27B LLM", fused-GEMM global-scale box and
# pipeline step (2): one shared global scale per fused group, member ratios
# folded into the E4M3 block scales, re-rounding at most ~6.2%.

def test_e4m3_round_nearest_matches_torch_and_ties_to_even():
    vals = F.E4M3_VALUES[:127]
    mids = (vals[:-1] + vals[1:]) / 2                       # exact midpoints (float64)
    rng = np.random.default_rng(311)
    ys = np.concatenate([vals, mids, rng.uniform(0, 448, 20000), 2.0 ** rng.uniform(-14, 8.8, 20000)])
    ys = np.minimum(ys.astype(np.float32).astype(np.float64), 448.0)
    got = F.e4m3_round_nearest(ys)
    want = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)
    # ties: the midpoint between bytes 0x40 (2.0) and 0x41 (2.25) goes to 0x40, 0x41..0x42 to 0x42
    assert F.e4m3_round_nearest(np.array([2.125]))[0] == 0x40
    assert F.e4m3_round_nearest(np.array([2.375]))[0] == 0x42


def test_harmonize_identity_power_of_two_and_bound():
    rng = np.random.default_rng(312)
    sb = rng.integers(0x08, 0x7F, (64, 32)).astype(np.uint8)           # normal E4M3 scales
    (same,), st = nvfp4.harmonize([sb], [np.float32(0.01)])
    np.testing.assert_array_equal(same, sb)
    # ratio 1/2: every normal scale >= 2^-5 halves exactly
    big = np.where(F.e4m3_decode(sb) >= 2.0 ** -5, sb, 0x30).astype(np.uint8)
    out, st = nvfp4.harmonize([big, big], [np.float32(0.5), np.float32(1.0)])
    np.testing.assert_array_equal(F.e4m3_decode(out[0]), F.e4m3_decode(big) / 2)
    np.testing.assert_array_equal(out[1], big)
    assert st == np.float32(1.0)
    # worst ratio of the page (2.81x): normal results within half an E4M3 step
    out, st = nvfp4.harmonize([sb], [np.float32(1.0 / 2.81)])
    out2, _ = nvfp4.harmonize([sb, sb], [np.float32(1.0 / 2.81), np.float32(1.0)])
    np.testing.assert_array_equal(out2[0], F.e4m3_round_nearest(
        (F.e4m3_decode(sb).astype(np.float32) * np.float32(np.float32(1.0 / 2.81) / np.float32(1.0))).astype(np.float64)))
    exact = F.e4m3_decode(sb) * np.float64(np.float32(np.float32(1.0 / 2.81) / np.float32(1.0)))
    got = F.e4m3_decode(out2[0])
    normal = exact >= 2.0 ** -6
    assert np.all(np.abs(got[normal] - exact[normal]) <= exact[normal] / 16 * (1 + 1e-9))


def test_harmonize_leaves_invalid_bytes_and_zero_scales():
    sb = np.array([[0x00, 0x7F, 0x80, 0xFE, 0xFF, 0x01, 0x7E]], dtype=np.uint8)
    (out,), st = nvfp4.harmonize([sb], [np.float32(0.25)])
    np.testing.assert_array_equal(out, sb)                       # ratio 1
    (out, _), st = nvfp4.harmonize([sb, sb], [np.float32(0.25), np.float32(1.0)])
    # 0 -> 0; invalid bytes untouched; 2^-9/4 -> 0; 448/4 = 112 = 1.75 * 2^6 -> 0x6E
    np.testing.assert_array_equal(out, np.array([[0x00, 0x7F, 0x80, 0xFE, 0xFF, 0x00, 0x6E]], np.uint8))
    # all members zero: the shared scale is 0 and nothing changes
    out, st = nvfp4.harmonize([sb, sb], [np.float32(0.0), np.float32(0.0)])
    assert st == 0 and all(np.array_equal(o, sb) for o in out)


def test_harmonized_fused_gemm_matches_separate_gemms():
    # the page's probe: a fused GEMM that takes the larger member scale
    # without rescaling is badly wrong; after harmonization it matches the
    # members' own GEMMs up to the re-rounding
    from oracle import gemm as G
    x = synth.heavy_tailed_f32(313, 314, (32, 256))
    w1 = synth.normal_f32(315, (48, 256), 0.02)
    w2 = synth.normal_f32(316, (48, 256), 0.02 / 2.75)          # member scales differ 2.75x
    cx, sx, tx = nvfp4.quantize(x)
    c1, s1, t1 = nvfp4.quantize(w1)
    c2, s2, t2 = nvfp4.quantize(w2)
    ref = np.concatenate([G.w4a4_nvfp4(cx, sx, tx, c1, s1, t1), G.w4a4_nvfp4(cx, sx, tx, c2, s2, t2)], axis=1)
    cw = np.concatenate([c1, c2])
    naive = G.w4a4_nvfp4(cx, sx, tx, cw, np.concatenate([s1, s2]), max(t1, t2))
    (h1, h2), st = nvfp4.harmonize([s1, s2], [t1, t2])
    fused = G.w4a4_nvfp4(cx, sx, tx, cw, np.concatenate([h1, h2]), st)
    assert G.rel_err(naive, ref)[0] > 0.3
    assert G.rel_err(fused, ref)[0] < 0.03
