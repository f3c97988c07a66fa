"""GPU parity past the 4 GiB operand limit: a 1,200,016 x 7168 weight (17 GB of
bf16, 4.3 GB of FP4 codes) goes through NVFP4 (dynamic scale) and MXFP4
quantization, the prefill, decode and W4A16 GEMMs, and a Sigma-Delta segment
of the same shape (fp32 master).  Those sizes take the
kernels' 64-bit addressing paths; the sampled rows include the last ones,
whose bytes lie beyond 4 GiB.  The weight is drawn on the device from a seeded
torch generator (8.6 G values would take minutes on the host); the oracle
reads the same rows back, so both sides see identical inputs."""
import numpy as np
import pytest
import torch

from oracle import formats as OF, nvfp4 as ONV, mxfp4 as OMX, gemm as OG, sigma_delta as OSD
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_bf16, host, packed, assert_bytes_equal

pytestmark = pytest.mark.gpu

N, K = 1_200_016, 7168              # N * K / 2 > 2^32 bytes of codes; K at the fused decode's maximum


def _rows():
    return np.array([0, 1, 4097, 599999, N - 17, N - 2, N - 1])


def _check(y, y_ref, what):
    whole, row, _ = OG.rel_err(y, y_ref)
    assert whole <= 1e-3 and row <= 1e-3, (what, whole, row)


def test_operands_past_4gib():
    L = fp4q()
    dev = "cuda:0"
    free, _ = torch.cuda.mem_get_info()
    if free < 40 << 30:
        pytest.skip("needs 40 GiB of free device memory")
    g = torch.Generator(device=dev)
    g.manual_seed(9001)
    w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, N, 65536):                       # fp32 draws in slices, stored as bf16
        r1 = min(N, r0 + 65536)
        w[r0:r1] = (torch.randn((r1 - r0, K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    rows = _rows()
    w_rows = w[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    wf = OF.bf16_bits_to_f32(w_rows)
    # exact max|w| without a 17 GB temporary: the larger magnitude of max and min
    amax = max(abs(float(w.max().float().cpu())), abs(float(w.min().float().cpu())))
    print("generated", flush=True)

    # NVFP4, dynamic tensor scale
    bc, bs, bt = L.quantize_nvfp4(w)
    tw = ONV.tensor_scale_from_amax(np.float32(amax))
    assert host(bt)[0] == tw
    cw, sw, _ = ONV.quantize(wf, tensor_scale=tw)
    idx = torch.from_numpy(rows).to(dev)
    assert_bytes_equal(host(bs[idx]), sw, "nvfp4 scales past 4 GiB")
    assert_bytes_equal(host(bc[idx]), packed(cw), "nvfp4 codes past 4 GiB")

    print("nvfp4 quantization checked", flush=True)
    # prefill NVFP4 GEMM (M = 64) and decode (M = 1, 2), sampled columns
    xb = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(9002, 9003, (64, K)))
    xf = OF.bf16_bits_to_f32(xb)
    xd = dev_bf16(xb)
    ac, as_, at = L.quantize_nvfp4(xd)
    cx, sx, tx = ONV.quantize(xf)
    assert host(at)[0] == tx
    y = L.gemm_w4a4(L.NVFP4, ac, as_, at, bc, bs, bt)
    _check(host(y[:, idx]), OG.w4a4_nvfp4(cx, sx, tx, cw, sw, tw), "nvfp4 gemm 64 x N")
    del y
    for M in (1, 2):
        yd, _ = L.linear_w4a4(xd[:M].contiguous(), bc, bs, bt)
        cxm, sxm, txm = ONV.quantize(xf[:M])
        _check(host(yd[:, idx]), OG.w4a4_nvfp4(cxm, sxm, txm, cw, sw, tw), f"decode M={M}")
    # W4A16 on the same weight (bf16 activation, NVFP4 weight)
    yw = L.gemm_w4a16(xd, bc, bs, bt)
    _check(host(yw[:, idx]), OG.w4a16(xb, cw, sw, tw), "w4a16 64 x N")
    del yw
    del bc, bs, bt
    torch.cuda.empty_cache()

    print("nvfp4 gemms checked", flush=True)
    # MXFP4 (rotation on) and its GEMM (M = 64)
    mc, ms = L.quantize_mxfp4(w, None, True)
    cwm, swm = OMX.quantize(OMX.hadamard32_scale(wf))
    assert_bytes_equal(host(ms[idx]), swm, "mxfp4 scales past 4 GiB")
    assert_bytes_equal(host(mc[idx]), packed(cwm), "mxfp4 codes past 4 GiB")
    del w
    torch.cuda.empty_cache()
    xc, xs = L.quantize_mxfp4(dev_bf16(xb), None, True)
    cxm, sxm = OMX.quantize(OMX.hadamard32_scale(xf))
    ym = L.gemm_w4a4(L.MXFP4, xc, xs, None, mc, ms, None)
    _check(host(ym[:, idx]), OG.w4a4_mxfp4(cxm, sxm, cwm, swm), "mxfp4 gemm 64 x N")
    del mc, ms, ym
    torch.cuda.empty_cache()


def test_sigma_delta_past_4gib():
    # one 1,200,016 x 7168 segment: fp32 master and residue of 34 GB each
    L = fp4q()
    dev = "cuda:0"
    free, _ = torch.cuda.mem_get_info()
    if free < 100 << 30:
        pytest.skip("needs 100 GiB of free device memory")
    g = torch.Generator(device=dev)
    g.manual_seed(9011)
    w = torch.empty((N, K), dtype=torch.float32, device=dev)
    for r0 in range(0, N, 65536):
        r1 = min(N, r0 + 65536)
        w[r0:r1] = torch.randn((r1 - r0, K), device=dev, generator=g) * 0.02
    rows = _rows()
    idx = torch.from_numpy(rows).to(dev)
    w_rows = host(w[idx])
    amax = max(abs(float(w.max().cpu())), abs(float(w.min().cpu())))
    c0, sc, ts = L.quantize_nvfp4(w)
    st = ONV.tensor_scale_from_amax(np.float32(amax))
    assert host(ts)[0] == st
    res = torch.zeros_like(w)
    codes = torch.empty_like(c0)
    del c0
    seg = [{"w": w, "scales": sc, "tensor_scale": ts, "residue": res, "codes": codes}]
    ref = OSD.sigma_delta_nvfp4(w_rows, 2, tensor_scale=st)
    assert_bytes_equal(host(sc[idx]), ref["scales"], "sigma-delta scales past 4 GiB")
    for k in range(2):
        L.sigma_delta_requant(seg, steps=1)
        assert_bytes_equal(host(codes[idx]), packed(ref["codes"][k]), f"sigma-delta codes, step {k + 1}")
        assert_bytes_equal(host(res[idx]).view(np.uint32), ref["residues"][k].view(np.uint32),
                           f"sigma-delta residues, step {k + 1}")
    del w, res, codes, sc, ts, seg
    torch.cuda.empty_cache()
