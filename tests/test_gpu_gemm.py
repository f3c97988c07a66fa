"""GPU parity of the GEMM kernels against the oracle's float64 product of the
exactly dequantized operands.  Bar: relative Frobenius error <= 1e-3 for the
whole matrix and for every row (the float64 oracle differs from the fp32
accumulation only by rounding, ~1e-7, so the bar catches any wrong term)."""
import numpy as np
import pytest
import torch

from oracle import formats as OF, nvfp4 as ONV, mxfp4 as OMX, balance as OBAL, sigma_delta as OSD, gemm as OG
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, dev_bf16, host, packed, assert_bytes_equal, sample_rows

pytestmark = pytest.mark.gpu
F32 = np.float32
TOL = 1e-3


def _check(y, y_ref, what, strict=1e-5):
    whole, row, mx = OG.rel_err(y, y_ref)
    print(f"{what}: rel err whole {whole:.3e} worst row {row:.3e} max {mx:.3e}")
    assert whole <= TOL and row <= TOL, (what, whole, row)
    # exact operands + fp32 accumulation: far inside the bar
    assert whole <= strict, (what, whole)


def _nv_gpu(x):
    return fp4q().quantize_nvfp4(x)


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (37, 200, 384), (130, 129, 128), (16, 300, 512),
                                   (1, 70, 256), (4, 64, 1024), (17, 64, 256)])
def test_nvfp4_gemm_small_ragged(M, N, K):
    x = synth.heavy_tailed_f32(200 + M, 201, (M, K))
    w = synth.normal_f32(202 + N, (N, K), 0.02)
    L = fp4q()
    ac, as_, at = _nv_gpu(dev_f32(x))
    bc, bs, bt = _nv_gpu(dev_f32(w))
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    cx, sx, tx = ONV.quantize(x)
    cw, sw, tw = ONV.quantize(w)
    _check(y, OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), f"nvfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nvfp4_tiny_config(seed):
    wl = synth.nvfp4_tiny(seed=seed)
    x, w = wl.arrays["x"], wl.arrays["w"]
    L = fp4q()
    ac, as_, at = _nv_gpu(dev_f32(x))
    bc, bs, bt = _nv_gpu(dev_f32(w))
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    cx, sx, tx = ONV.quantize(x)
    cw, sw, tw = ONV.quantize(w)
    _check(y, OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), f"nvfp4 tiny config, input set {seed}")


def test_nvfp4_gemm_wide_tiles_ragged():
    # 4000 x 10100 takes the 320-wide tiles (two full rounds) with partial
    # tiles in both M and N; sampled rows include the last ones
    L = fp4q()
    x = synth.heavy_tailed_f32(210, 211, (4000, 256))
    w = synth.normal_f32(212, (10100, 256), 0.02)
    ac, as_, at = _nv_gpu(dev_f32(x))
    bc, bs, bt = _nv_gpu(dev_f32(w))
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    rows, cols = sample_rows(4000, 40, 3), sample_rows(10100, 400, 4)
    cx, sx, tx = ONV.quantize(x)
    cw, sw, tw = ONV.quantize(w)
    ref = OG.w4a4_nvfp4(cx[rows], sx[rows], tx, cw[cols], sw[cols], tw)
    _check(y[np.ix_(rows, cols)], ref, "nvfp4 4000x10100x256 (320-wide tiles)")


def test_nvfp4_prefill_full_size_sampled():
    wl = synth.nvfp4_prefill()
    xb, wb = wl.arrays["x_bf16"], wl.arrays["w_bf16"]
    L = fp4q()
    ac, as_, at = _nv_gpu(dev_bf16(xb))
    bc, bs, bt = _nv_gpu(dev_bf16(wb))
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    assert np.isfinite(y).all()
    xf, wf = OF.bf16_bits_to_f32(xb), OF.bf16_bits_to_f32(wb)
    rows, cols = sample_rows(4096, 40, 1), sample_rows(10240, 300, 2)
    tx = ONV.tensor_scale_from_amax(np.abs(xf).max())
    tw = ONV.tensor_scale_from_amax(np.abs(wf).max())
    cx, sx, _ = ONV.quantize(xf[rows], tensor_scale=tx)
    cw, sw, _ = ONV.quantize(wf[cols], tensor_scale=tw)
    _check(y[np.ix_(rows, cols)], OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), "nvfp4 prefill 4096x10240x5120 (sampled)")


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (200, 130, 384), (5, 17, 128)])
def test_mxfp4_gemm_small_ragged(M, N, K):
    x = synth.heavy_tailed_f32(210 + M, 211, (M, K))
    w = synth.normal_f32(212 + N, (N, K), 0.02)
    L = fp4q()
    ac, as_ = L.quantize_mxfp4(dev_f32(x), None, True)
    bc, bs = L.quantize_mxfp4(dev_f32(w), None, True)
    y = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, bc, bs, None))
    cx, sx = OMX.quantize(OMX.hadamard32_scale(x))
    cw, sw = OMX.quantize(OMX.hadamard32_scale(w))
    _check(y, OG.w4a4_mxfp4(cx, sx, cw, sw), f"mxfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2048, 8192, 256), (200, 300, 512)])
def test_mxfp4_gemm_both_column_tiles(M, N, K):
    # the launcher picks the column tile by rounds over the compute units:
    # 2048 x 8192 fills one round with 256-wide tiles (224 would need two),
    # which run on 32 x 32 x 64 instructions; 200 x 300 takes 224-wide tiles
    # on 16 x 16 x 128, ragged in both M and N
    x = synth.heavy_tailed_f32(220 + M, 221, (M, K))
    w = synth.normal_f32(222 + N, (N, K), 0.02)
    L = fp4q()
    ac, as_ = L.quantize_mxfp4(dev_f32(x), None, True)
    bc, bs = L.quantize_mxfp4(dev_f32(w), None, True)
    y = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, bc, bs, None))
    rows, cols = sample_rows(M, 40, 5), sample_rows(N, 200, 6)
    cx, sx = OMX.quantize(OMX.hadamard32_scale(x[rows]))
    cw, sw = OMX.quantize(OMX.hadamard32_scale(w[cols]))
    _check(y[np.ix_(rows, cols)], OG.w4a4_mxfp4(cx, sx, cw, sw), f"mxfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(768, 22400, 128), (600, 25000, 384), (1000, 30000, 256), (300, 9000, 1152),
                                   (1000, 30000, 1024)])
def test_mxfp4_gemm_many_tiles_ragged(M, N, K):
    # more output tiles than compute units, partial tiles in M and N, and K
    # that is (1000 x 30000 x 256 and x 1024) or is not (K = 128, 384, 1152)
    # a whole number of the direct-load kernel's 256-element stages; the
    # 1000 x 30000 shapes take 256-wide tiles, with one stage (K = 256) and
    # with four (K = 1024)
    x = synth.heavy_tailed_f32(230 + M, 231, (M, K))
    w = synth.normal_f32(232 + K, (N, K), 0.02)
    L = fp4q()
    ac, as_ = L.quantize_mxfp4(dev_f32(x), None, True)
    bc, bs = L.quantize_mxfp4(dev_f32(w), None, True)
    y = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, bc, bs, None))
    assert np.isfinite(y).all()
    rows, cols = sample_rows(M, 40, 7), sample_rows(N, 300, 8)
    cx, sx = OMX.quantize(OMX.hadamard32_scale(x[rows]))
    cw, sw = OMX.quantize(OMX.hadamard32_scale(w[cols]))
    _check(y[np.ix_(rows, cols)], OG.w4a4_mxfp4(cx, sx, cw, sw), f"mxfp4 {M}x{N}x{K} (many tiles)")


def test_mxfp4_gemm_strided_output():
    # ldy > N with ldy % 4 != 0: the output leaves through the masked path
    L = fp4q()
    M, N, K, ldy = 300, 500, 256, 503
    x = synth.heavy_tailed_f32(240, 241, (M, K))
    w = synth.normal_f32(242, (N, K), 0.02)
    ac, as_ = L.quantize_mxfp4(dev_f32(x), None, True)
    bc, bs = L.quantize_mxfp4(dev_f32(w), None, True)
    yb = torch.full((M, ldy), 7.0, dtype=torch.float32, device="cuda:0")
    L.gemm_w4a4(L.MXFP4, ac, as_, None, bc, bs, None, out=yb[:, :N])
    y = host(yb)
    assert (y[:, N:] == 7.0).all(), "columns past N were written"
    cx, sx = OMX.quantize(OMX.hadamard32_scale(x))
    cw, sw = OMX.quantize(OMX.hadamard32_scale(w))
    _check(y[:, :N], OG.w4a4_mxfp4(cx, sx, cw, sw), "mxfp4 300x500x256 ldy 503")


def test_mxfp4_transform_full_size_sampled():
    wl = synth.mxfp4_transform()
    xb, wb = wl.arrays["x_bf16"], wl.arrays["w_bf16"]
    xf, wf = OF.bf16_bits_to_f32(xb), OF.bf16_bits_to_f32(wb)
    _, t32, u32 = OBAL.balance_scale(wf, xf)
    L = fp4q()
    ac, as_ = L.quantize_mxfp4(dev_bf16(xb), dev_f32(t32), True)
    bc, bs = L.quantize_mxfp4(dev_bf16(wb), dev_f32(u32), True)
    y = host(L.gemm_w4a4(L.MXFP4, ac, as_, None, bc, bs, None))
    assert np.isfinite(y).all()
    rows, cols = sample_rows(2048, 40, 3), sample_rows(14336, 300, 4)
    cx, sx = OMX.quantize(OMX.hadamard32_scale(xf[rows], t32))
    cw, sw = OMX.quantize(OMX.hadamard32_scale(wf[cols], u32))
    y_ref = OG.w4a4_mxfp4(cx, sx, cw, sw)
    _check(y[np.ix_(rows, cols)], y_ref, "mxfp4 2048x14336x4096 (sampled)")
    # the transform leaves the unquantized product unchanged, so the W4A4
    # result approximates X W^T (sanity, not parity)
    ref = xf[rows].astype(np.float64) @ wf[cols].astype(np.float64).T
    assert OG.rel_err(y_ref, ref)[0] < 0.3


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (130, 200, 384), (4096, 768, 768)])
def test_w4a16_gemm(M, N, K):
    a = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(220 + M, 221, (M, K)))
    w = synth.normal_f32(222 + N, (N, K), 0.02)
    L = fp4q()
    bc, bs, bt = _nv_gpu(dev_f32(w))
    y = host(L.gemm_w4a16(dev_bf16(a), bc, bs, bt))
    cw, sw, tw = ONV.quantize(w)
    rows = sample_rows(M, 64, 5)
    _check(y[rows], OG.w4a16(a[rows], cw, sw, tw), f"w4a16 {M}x{N}x{K}")


def test_w4a16_on_sigma_delta_codes():
    wl = synth.looped_sigma_delta(tokens=512)
    w = wl.arrays["w6"]                       # down projection 768 x 3072
    hd = wl.arrays["hd_bf16"]
    L = fp4q()
    wd = dev_f32(w)
    c0, sc, ts = L.quantize_nvfp4(wd)
    codes = torch.empty_like(c0)
    res = torch.zeros_like(wd)
    seg = [{"w": wd, "scales": sc, "tensor_scale": ts, "residue": res, "codes": codes}]
    ref = OSD.sigma_delta_nvfp4(w, 3)
    for k in range(3):
        L.sigma_delta_requant(seg, steps=1)
        y = host(L.gemm_w4a16(dev_bf16(hd), codes, sc, ts))
        _check(y, OG.w4a16(hd, ref["codes"][k], ref["scales"], ref["s_t"]), f"w4a16 sigma-delta step {k + 1}")


def test_decode_fused_equals_unfused_and_oracle():
    wl = synth.nvfp4_decode()
    xb, w = wl.arrays["x_bf16"], wl.arrays["w"]
    L = fp4q()
    bc, bs, bt = _nv_gpu(dev_f32(w))
    cw, sw, tw = ONV.quantize(w)
    assert_bytes_equal(host(bc), packed(cw), "decode weight codes")
    Wd = ONV.dequantize(cw, sw, tw)
    for M in (1, 2, 3, 4, 5, 16):
        xd = dev_bf16(xb[:M])
        y_f, ts_f = L.linear_w4a4(xd, bc, bs, bt)
        ac, as_, at = L.quantize_nvfp4(xd)
        y_u = L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt)
        y_f, y_u = host(y_f), host(y_u)
        assert host(ts_f)[0] == host(at)[0]
        assert_bytes_equal(y_f.view(np.uint32), y_u.view(np.uint32), f"fused vs unfused M={M}")
        xf = OF.bf16_bits_to_f32(xb[:M])
        cx, sx, tx = ONV.quantize(xf)
        assert host(at)[0] == tx
        y_ref = ONV.dequantize(cx, sx, tx) @ Wd.T
        _check(y_f, y_ref, f"decode M={M}")
        # static activation scale path
        y_s, _ = L.linear_w4a4(xd, bc, bs, bt, a_tscale=at)
        assert_bytes_equal(host(y_s).view(np.uint32), y_f.view(np.uint32), f"static scale M={M}")


@pytest.mark.parametrize("N,K", [(77, 384), (33, 7168), (130, 640), (1000, 512), (4100, 5120), (300, 2560)])
def test_decode_ragged(N, K):
    # ragged output count, short rows (fewer 16-byte chunks than lanes), the
    # longest supported row, and for the streamed form: row ranges that end
    # inside a 16-row group, its largest K (5120) and uneven load splits
    L = fp4q()
    w = synth.normal_f32(250 + N, (N, K), 0.02)
    x = synth.heavy_tailed_f32(251 + N, 252 + N, (16, K))
    xb = synth.f32_to_bf16_bits(x)
    bc, bs, bt = _nv_gpu(dev_f32(w))
    cw, sw, tw = ONV.quantize(w)
    for M in (1, 2, 3, 4, 5, 9, 16):
        yf, tf = L.linear_w4a4(dev_bf16(xb[:M]), bc, bs, bt)
        ac, as_, at = L.quantize_nvfp4(dev_bf16(xb[:M]))
        yu = L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt)
        assert_bytes_equal(host(yf).view(np.uint32), host(yu).view(np.uint32), f"fused vs unfused N={N} K={K} M={M}")
        cx, sx, tx = ONV.quantize(OF.bf16_bits_to_f32(xb[:M]))
        _check(host(yf), OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), f"decode N={N} K={K} M={M}")


@pytest.mark.parametrize("K", [32, 96, 160, 4128])
def test_gemm_k_multiple_of_32(K):
    # K needs only to be a multiple of 32 (one MXFP4 block): K % 128 != 0
    # runs on the register-staged kernels, whose last K stage is partly
    # empty (zero codes with zero scales; the scale words of a row are then
    # read byte by byte).  Every GEMM form, against the oracle.
    M, N = 70, 130
    x = synth.heavy_tailed_f32(260 + K, 261, (M, K))
    w = synth.normal_f32(262 + K, (N, K), 0.02)
    L = fp4q()
    print(f"K = {K}", flush=True)
    # NVFP4 prefill
    ac, as_, at = _nv_gpu(dev_f32(x))
    bc, bs, bt = _nv_gpu(dev_f32(w))
    cx, sx, tx = ONV.quantize(x)
    cw, sw, tw = ONV.quantize(w)
    _check(host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt)), OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw),
           f"nvfp4 {M}x{N}x{K}")
    # MXFP4 prefill
    mc, ms = L.quantize_mxfp4(dev_f32(x), None, True)
    nc, ns = L.quantize_mxfp4(dev_f32(w), None, True)
    rc, rs = OMX.quantize(OMX.hadamard32_scale(x))
    qc, qs = OMX.quantize(OMX.hadamard32_scale(w))
    _check(host(L.gemm_w4a4(L.MXFP4, mc, ms, None, nc, ns, None)), OG.w4a4_mxfp4(rc, rs, qc, qs),
           f"mxfp4 {M}x{N}x{K}")
    # W4A16
    xb = synth.f32_to_bf16_bits(x)
    _check(host(L.gemm_w4a16(dev_bf16(xb), bc, bs, bt)), OG.w4a16(xb, cw, sw, tw), f"w4a16 {M}x{N}x{K}")
    # decode: row-streamed (M <= 4) and register-staged (M > 4) forms, fused
    # and unfused, bit for bit with each other
    for m in (1, 3, 8, 16):
        yf, tf = L.linear_w4a4(dev_bf16(xb[:m]), bc, bs, bt)
        a2, s2, t2 = L.quantize_nvfp4(dev_bf16(xb[:m]))
        yu = L.gemm_w4a4(L.NVFP4, a2, s2, t2, bc, bs, bt)
        assert_bytes_equal(host(yf).view(np.uint32), host(yu).view(np.uint32), f"fused vs unfused K={K} M={m}")
        cxm, sxm, txm = ONV.quantize(OF.bf16_bits_to_f32(xb[:m]))
        _check(host(yf), OG.w4a4_nvfp4(cxm, sxm, txm, cw, sw, tw), f"decode K={K} M={m}")


def test_gemm_zero_and_one_hot():
    L = fp4q()
    K, N = 256, 64
    w = synth.normal_f32(230, (N, K), 0.02)
    bc, bs, bt = _nv_gpu(dev_f32(w))
    z = np.zeros((20, K), F32)
    ac, as_, at = _nv_gpu(dev_f32(z))
    assert not host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt)).any()
    e = np.zeros((20, K), F32)
    e[np.arange(20), np.arange(20) * 7] = 1.0
    ac, as_, at = _nv_gpu(dev_f32(e))
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    cw, sw, tw = ONV.quantize(w)
    ce, se, te = ONV.quantize(e)
    y_ref = OG.w4a4_nvfp4(ce, se, te, cw, sw, tw)
    assert np.array_equal(y.astype(np.float64), y_ref.astype(F32).astype(np.float64)) or OG.rel_err(y, y_ref)[0] < 1e-6


@pytest.mark.parametrize("M", [3, 40])
def test_nvfp4_gemm_subnormal_block_scales(M):
    # blocks far below the tensor maximum get E4M3 block scales in the
    # subnormal range (scale bytes 0x01..0x07); the GEMMs must dequantize them
    # exactly
    K, N = 512, 96
    rng = np.random.default_rng(240)
    x = rng.standard_normal((M, K)).astype(F32)
    x[:, :16] *= 1e5                                   # sets the tensor maximum
    for j, f in enumerate([1e-1, 3e-2, 1e-2, 3e-3, 1e-3, 3e-4]):
        x[:, 16 * (j + 1):16 * (j + 2)] *= f
    w = synth.normal_f32(241, (N, K), 0.02)
    w[:, 32:48] *= 1e-4
    L = fp4q()
    ac, as_, at = _nv_gpu(dev_f32(x))
    bc, bs, bt = _nv_gpu(dev_f32(w))
    cx, sx, tx = ONV.quantize(x)
    cw, sw, tw = ONV.quantize(w)
    assert (sx[:, 1:7] < 8).any() and (sx[:, 1:7] > 0).any()       # subnormal scales present
    y = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt))
    _check(y, OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), f"nvfp4 subnormal scales M={M}")
    if M <= 16:
        xb = synth.f32_to_bf16_bits(x)
        yf, _ = L.linear_w4a4(dev_bf16(xb), bc, bs, bt)
        cxb, sxb, txb = ONV.quantize(OF.bf16_bits_to_f32(xb))
        _check(host(yf), OG.w4a4_nvfp4(cxb, sxb, txb, cw, sw, tw), f"decode subnormal scales M={M}")


def test_w4a16_grouped_equals_single_launches():
    # the looped core's 13 linears at one loop step (hidden and the wider
    # down-projection input) plus ragged problems; one grouped call gives
    # the bytes of the 13 + 3 single calls
    L = fp4q()
    wl = synth.looped_sigma_delta(tokens=8)
    h = dev_bf16(wl.arrays["h_bf16"])
    hd = dev_bf16(wl.arrays["hd_bf16"])
    probs = []
    for i, (n, k) in enumerate(wl.meta["shapes"]):
        c, sc, ts = L.quantize_nvfp4(dev_f32(wl.arrays[f"w{i}"]))
        probs.append(((hd if k == 3072 else h), c, sc, ts))
    for M, N, K in ((130, 200, 384), (1, 70, 256), (64, 256, 1024)):
        a = dev_bf16(synth.f32_to_bf16_bits(synth.heavy_tailed_f32(700 + M, 701, (M, K))))
        c, sc, ts = L.quantize_nvfp4(dev_f32(synth.normal_f32(702 + N, (N, K), 0.02)))
        probs.append((a, c, sc, ts))
    print(f"grouped W4A16: {len(probs)} problems", flush=True)
    got = [host(y) for y in L.gemm_w4a16_grouped(probs)]
    for i, pr in enumerate(probs):
        want = host(L.gemm_w4a16(*pr))
        assert np.array_equal(got[i].view(np.uint32), want.view(np.uint32)), f"problem {i}"
    # and one of them against the oracle
    a, c, sc, ts = probs[-3]
    xb = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(830, 701, (130, 384)))
    w = synth.normal_f32(902, (200, 384), 0.02)
    cw, sw, tw = ONV.quantize(w)
    ref = OG.matmul_nt(OF.bf16_bits_to_f32(xb).astype(np.float64), ONV.dequantize(cw, sw, tw))
    _check(got[-3], ref, "grouped W4A16 130x200x384")


def test_w4a16_grouped_spans_several_launches():
    # 37 problems: more than one grouped launch holds (16 per launch), with
    # mixed K (launch order is longest K first) and ragged M, N
    L = fp4q()
    rng = np.random.default_rng(950)
    probs = []
    for i in range(37):
        M = int(rng.integers(1, 300))
        N = int(rng.integers(1, 20)) * 32 + int(rng.integers(0, 2)) * 7
        K = int(rng.choice([128, 256, 384, 768, 1024]))
        a = dev_bf16(synth.f32_to_bf16_bits(synth.heavy_tailed_f32(960 + i, 961, (M, K))))
        c, sc, ts = L.quantize_nvfp4(dev_f32(synth.normal_f32(962 + i, (N, K), 0.02)))
        probs.append((a, c, sc, ts))
    print(f"grouped W4A16: {len(probs)} problems in {(len(probs) + 15) // 16} launches", flush=True)
    got = [host(y) for y in L.gemm_w4a16_grouped(probs)]
    for i, pr in enumerate(probs):
        want = host(L.gemm_w4a16(*pr))
        assert np.array_equal(got[i].view(np.uint32), want.view(np.uint32)), f"problem {i}"
