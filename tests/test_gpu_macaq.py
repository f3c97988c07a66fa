"""GPU parity of the MACaQ weight-side refinement ("MACaQ: Fast, Model
Agnostic Calibrated Quantization for Low-Precision Weights and
Activations", "Core method" (iii)-(iv), "Method steps" 0, 3, 4) against the
oracle, through the C ABI: the Hessian, the screened exponents, the refined
codes and the flip counts must be bit-identical; the refined weight must
lower the W4A4 GEMM error on the calibration activations."""
import numpy as np
import pytest
import torch

from oracle import macaq as OMQ, mxfp4 as OMX, formats as OF
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, host, packed, assert_bytes_equal, sample_rows

pytestmark = pytest.mark.gpu
F32, F64 = np.float32, np.float64


def _correlated_x(seed, t, n):
    x = synth.normal_f32(seed, (t, n))
    x[:, 1:] = (0.8 * x[:, :-1] + 0.6 * x[:, 1:]).astype(F32)
    return x


def test_hessian_ragged_accumulating_chunks():
    L = fp4q()
    x = synth.heavy_tailed_f32(600, 601, (75, 72))
    h0 = synth.normal_f32(602, (72, 72)).astype(F64)
    print("hessian 75 x 72, two chunks", flush=True)
    h = torch.from_numpy(h0.copy()).cuda()
    xd = dev_f32(x)
    L.hessian_accumulate(xd[:37], h)
    L.hessian_accumulate(xd[37:], h)
    np.testing.assert_array_equal(host(h), OMQ.hessian(x, h0))
    # a strided view (48 of 72 columns)
    hs = L.hessian_accumulate(xd[:, :48])
    np.testing.assert_array_equal(host(hs), OMQ.hessian(np.ascontiguousarray(x[:, :48])))


def test_hessian_full_size_sampled_entries():
    # calibration rows of the MXFP4 layer (2048 tokens x 4096), transformed
    L = fp4q()
    x = synth.heavy_tailed_f32(3001, 3003, (2048, 4096))
    print("hessian 2048 x 4096", flush=True)
    h = host(L.hessian_accumulate(dev_f32(x)))
    rng = np.random.default_rng(603)
    j = np.concatenate([[0, 4095, 17], rng.integers(0, 4096, 300)])
    k = np.concatenate([[0, 4095, 4094], rng.integers(0, 4096, 300)])
    acc = np.zeros(j.size, F64)
    x64 = x.astype(F64)
    for t in range(x.shape[0]):                                 # tokens in order
        acc = acc + x64[t, j] * x64[t, k]
    np.testing.assert_array_equal(h[j, k], acc)
    np.testing.assert_array_equal(h, h.T)


def _refine_check(w, x, k_iters, rows=None, lam=1.0):
    L = fp4q()
    h = OMQ.hessian(x)
    hd_gpu = L.hessian_accumulate(dev_f32(x))
    np.testing.assert_array_equal(host(hd_gpu), h)
    print(f"macaq refine {w.shape}, K={k_iters}", flush=True)
    codes, scales, flips = L.macaq_refine(dev_f32(w), hd_gpu, lam, k_iters)
    codes, scales, flips = host(codes), host(scales), host(flips)
    sel = np.arange(w.shape[0]) if rows is None else rows
    c_ref, s_ref, f_ref = OMQ.refine(w[sel], h, lam, k_iters)
    assert_bytes_equal(scales[sel], s_ref, "screened exponents")
    assert_bytes_equal(codes[sel], packed(c_ref), "refined codes")
    np.testing.assert_array_equal(flips[sel], f_ref)
    return codes, scales, flips


def test_refine_small_ragged_bit_exact():
    x = _correlated_x(604, 256, 320)
    w = synth.normal_f32(605, (70, 320), 0.02)
    w[3] = 0.0                                     # an all-zero row
    w[5, 32:64] = 0.0                              # an all-zero block
    w[6, :32] = -0.0                               # negative zeros
    w[6, 7] = 1e-3
    w[7, 64:96] *= 1e-30                           # tiny block (exponent near the low end)
    w[8, 96:128] *= 1e30                           # huge block
    for k in (0, 3, 128):
        codes, scales, flips = _refine_check(w, x, k)
    assert flips.sum() > 0 and flips[3] == 0


@pytest.mark.parametrize("n", [4128, 8224])
def test_refine_wide_rows(n):
    # rows wider than 4096 (512 threads per row) and than 8192 (1024)
    x = _correlated_x(620 + n % 7, 16, n)
    w = synth.heavy_tailed_f32(621, 622, (5, n))
    _refine_check(w, x, 128)


def test_refine_ridge_factor_and_row_stride():
    L = fp4q()
    x = _correlated_x(606, 128, 256)
    w = synth.heavy_tailed_f32(607, 608, (40, 288))
    h = OMQ.hessian(x)
    wd = dev_f32(w)[:, :256]                       # ldw 288
    codes, scales, flips = L.macaq_refine(wd, torch.from_numpy(h).cuda(), 0.25, 20)
    c_ref, s_ref, f_ref = OMQ.refine(np.ascontiguousarray(w[:, :256]), h, 0.25, 20)
    assert_bytes_equal(host(scales), s_ref, "exponents, lambda 0.25")
    assert_bytes_equal(host(codes), packed(c_ref), "codes, lambda 0.25")
    np.testing.assert_array_equal(host(flips), f_ref)


def test_refine_full_size_sampled_rows():
    # the MXFP4 layer's weight (14336 x 4096) with a 64-token Hessian
    w = synth.normal_f32(3002, (14336, 4096), 0.02)
    x = synth.heavy_tailed_f32(3001, 3003, (64, 4096))
    rows = sample_rows(14336, 6, 609)
    _refine_check(w, x, 128, rows=rows)


def test_refined_weight_lowers_the_gemm_error():
    # the layer end to end: balance scale + Hadamard on both sides, MXFP4
    # activations, weight refined on the calibration rows; the refined weight
    # brings the W4A4 product closer to the exact X W^T than the plain
    # nearest-code weight
    L = fp4q()
    x = _correlated_x(610, 512, 1024)
    x[:, synth.outlier_columns(611, 1024, 10)] *= 32.0
    w = synth.normal_f32(612, (256, 1024), 0.02)
    xd, wd = dev_f32(x), dev_f32(w)
    t, u = L.balance_scale(wd, xd)
    xp, wp = L.hadamard32_scale(xd, t), L.hadamard32_scale(wd, u)
    h = L.hessian_accumulate(xp)
    ac, as_ = L.quantize_mxfp4(xd, t, True)
    rc, rs = L.quantize_mxfp4(wd, u, True)
    qc, qs, flips = L.macaq_refine(wp, h, 1.0, 128)
    y_rtn = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, rc, rs, None)).astype(F64)
    y_ref = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, qc, qs, None)).astype(F64)
    y = x.astype(F64) @ w.astype(F64).T
    e_rtn = np.linalg.norm(y_rtn - y) / np.linalg.norm(y)
    e_ref = np.linalg.norm(y_ref - y) / np.linalg.norm(y)
    print(f"W4A4 relative error: nearest codes {e_rtn:.4f}, refined {e_ref:.4f}, flips {host(flips).sum()}")
    assert e_ref < 0.85 * e_rtn                    # the oracle on these inputs: 0.094 -> 0.068
