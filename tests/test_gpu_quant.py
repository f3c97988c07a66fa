"""GPU parity of the quantization kernels against the CPU oracle, through
the C ABI: codes, block scales, tensor scales, rotated values and
Sigma-Delta residues must be bit-identical."""
import zlib

import numpy as np
import pytest
import torch

from oracle import formats as OF, nvfp4 as ONV, mxfp4 as OMX, balance as OBAL, sigma_delta as OSD
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, dev_bf16, host, packed, assert_bytes_equal, sample_rows

pytestmark = pytest.mark.gpu
F32 = np.float32


def _nv_check(x_f32_host, x_dev, tensor_scale=None, rows=None, rule="6"):
    L = fp4q()
    ts_in = None if tensor_scale is None else dev_f32(np.array([tensor_scale], F32))
    codes, scales, ts = L.quantize_nvfp4(x_dev, tensor_scale=ts_in, rule=rule)
    codes, scales, ts = host(codes), host(scales), host(ts)
    st_ref = ONV.tensor_scale_from_amax(np.abs(x_f32_host).max()) if tensor_scale is None else F32(tensor_scale)
    assert ts[0] == st_ref, (ts[0], st_ref)
    sel = np.arange(x_f32_host.shape[0]) if rows is None else rows
    c_ref, s_ref, _ = ONV.quantize(x_f32_host[sel], tensor_scale=st_ref, rule=rule)
    assert_bytes_equal(scales[sel], s_ref, "nvfp4 scales")
    assert_bytes_equal(codes[sel], packed(c_ref), "nvfp4 codes")


def test_abi_version_and_device():
    assert fp4q().abi_version() == 1


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nvfp4_tiny_config_bit_exact(seed):
    wl = synth.nvfp4_tiny(seed=seed)
    for name in ("x", "w"):
        a = wl.arrays[name]
        _nv_check(a, dev_f32(a))


def test_nvfp4_ragged_strided_bf16_and_static_scale():
    x = synth.heavy_tailed_f32(101, 102, (37, 96))
    xb = synth.f32_to_bf16_bits(x)
    xf = OF.bf16_bits_to_f32(xb)
    # strided view: 80 of 96 columns
    full = dev_bf16(xb)
    _nv_check(np.ascontiguousarray(xf[:, :80]), full[:, :80])
    _nv_check(xf, full, tensor_scale=F32(0.0123))
    _nv_check(x, dev_f32(x))


def test_nvfp4_edge_values():
    x = synth.normal_f32(103, (8, 64))
    x[0, :16] = 0.0                      # zero block
    x[1, :] = -0.0                       # negative zeros in a row
    x[1, 3] = 1e-3
    x[2, :16] = np.float32(3e38)         # huge block
    x[3, :16] = np.float32(1e-42)        # subnormal block
    x[4, 5] = np.float32(-7e-45)
    _nv_check(x, dev_f32(x))
    z = np.zeros((4, 32), F32)
    _nv_check(z, dev_f32(z))


def test_nvfp4_e4m3_ceil_sweep():
    # s_t = fl(1/6) makes fl(6 * s_t) == 1, so each block's scale input is
    # its maximum exactly; sweep maxima around every E4M3 value
    st = F32(1.0) / F32(6.0)
    assert F32(F32(6) * st) == 1.0
    table = OF.E4M3_VALUES[:127]
    amax = []
    for v in table[1:]:
        b = np.array([v], F32).view(np.int32)[0]
        for d in (-2, -1, 0, 1, 2):
            amax.append(np.array([b + d], np.int32).view(F32)[0])
    amax += [F32(449.0), F32(1e-5), F32(2.0 ** -10), F32(3e-45)]
    amax = np.array(amax, F32)
    n = len(amax) - len(amax) % 4
    rng = np.random.default_rng(104)
    x = (rng.uniform(-1, 1, (n, 16)).astype(F32) * amax[:n, None]).astype(F32)
    x[np.arange(n), rng.integers(0, 16, n)] = amax[:n]
    x = x.reshape(n // 4, 64)
    _nv_check(x, dev_f32(x), tensor_scale=st)


def test_nvfp4_prefill_full_size_sampled_rows():
    wl = synth.nvfp4_prefill()
    for name in ("x_bf16", "w_bf16"):
        b = wl.arrays[name]
        xf = OF.bf16_bits_to_f32(b)
        _nv_check(xf, dev_bf16(b), rows=sample_rows(b.shape[0], seed=zlib.crc32(name.encode()) % 1000))


def test_nvfp46_tiny_ragged_strided_and_static():
    # 4/6 block scales: same inputs as the max -> 6 tests, bit-exact
    wl = synth.nvfp4_tiny()
    for name in ("x", "w"):
        a = wl.arrays[name]
        _nv_check(a, dev_f32(a), rule="4/6")
    x = synth.heavy_tailed_f32(401, 402, (37, 96))
    xb = synth.f32_to_bf16_bits(x)
    xf = OF.bf16_bits_to_f32(xb)
    full = dev_bf16(xb)
    _nv_check(np.ascontiguousarray(xf[:, :80]), full[:, :80], rule="4/6")
    _nv_check(xf, full, tensor_scale=F32(0.0123), rule="4/6")
    _nv_check(x, dev_f32(x), rule="4/6")


def test_nvfp46_edge_values_and_exact_blocks():
    x = synth.normal_f32(403, (8, 64))
    x[0, :16] = 0.0                      # zero block
    x[1, :] = -0.0
    x[1, 3] = 1e-3
    x[2, :16] = np.float32(3e38)         # huge block (errors overflow to inf: tie -> 6)
    x[3, :16] = np.float32(1e-42)        # subnormal block
    x[4, 5] = np.float32(-7e-45)
    _nv_check(x, dev_f32(x), rule="4/6")
    # blocks exactly representable under exactly one candidate (s_t = 1/16)
    four = [4, 2, 1, 0.5, 1.5, 3, 0, -4, -2, -1, -0.5, -1.5, -3, 0, 4, 2]
    six = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, 0]
    e = np.array([four + six] * 4, F32)
    _nv_check(e, dev_f32(e), tensor_scale=F32(0.0625), rule="4/6")


def test_nvfp46_prefill_full_size_sampled_rows():
    wl = synth.nvfp4_prefill()
    for name in ("x_bf16", "w_bf16"):
        b = wl.arrays[name]
        xf = OF.bf16_bits_to_f32(b)
        _nv_check(xf, dev_bf16(b), rows=sample_rows(b.shape[0], seed=zlib.crc32(name.encode()) % 1000 + 7), rule="4/6")


def test_sigma_delta_on_46_scales():
    # the looped core's chain with the 4/6 block scales of the section 2.5
    # listing: codes and residues bit-exact over several steps
    L = fp4q()
    w = synth.normal_f32(404, (96, 768), 0.02)
    wd = dev_f32(w)
    _, sc, ts = L.quantize_nvfp4(wd, rule="4/6")
    codes = torch.empty((96, 384), dtype=torch.uint8, device="cuda:0")
    res = torch.zeros_like(wd)
    seg = [{"w": wd, "scales": sc, "tensor_scale": ts, "residue": res, "codes": codes}]
    ref = OSD.sigma_delta_nvfp4(w, 5, rule="4/6")
    assert_bytes_equal(host(sc), ref["scales"], "4/6 scales")
    for k in range(5):
        L.sigma_delta_requant(seg, steps=1)
        assert_bytes_equal(host(codes), packed(ref["codes"][k]), f"codes step {k + 1}")
        assert_bytes_equal(host(res).view(np.uint32), ref["residues"][k].view(np.uint32), f"residue step {k + 1}")


def test_nvfp4_dynamic_large_tensor():
    # 8192 x 7168 bf16 (58.7 M elements): the amax pass runs at its largest
    # grid, and the partial maxima fill the front of the block-scale buffer
    b = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(105, 106, (8192, 7168)))
    xf = OF.bf16_bits_to_f32(b)
    _nv_check(xf, dev_bf16(b), rows=sample_rows(b.shape[0], seed=7))


def _nv_ref(x_f32_host):
    """Oracle codes, scales and tensor scale as device tensors."""
    st = ONV.tensor_scale_from_amax(np.abs(x_f32_host).max())
    c, sc, _ = ONV.quantize(x_f32_host, tensor_scale=st)
    return (torch.from_numpy(packed(c)).to("cuda:0"), torch.from_numpy(np.ascontiguousarray(sc)).to("cuda:0"),
            torch.tensor([st], dtype=torch.float32, device="cuda:0"))


def _same(got, want):
    return all(torch.equal(g, w) for g, w in zip(got, want))


def test_nvfp4_dynamic_repeated_calls_streams_and_graph():
    """Dynamic quantization many times in a row, from two side streams
    without host synchronisation, and replayed from a captured graph with
    the input changed between replays (the amax, finalize and quantize
    launches all go into the graph): every result must equal the oracle's."""
    L = fp4q()
    ba = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(111, 112, (48, 160)))        # one workgroup
    bb = synth.f32_to_bf16_bits(synth.heavy_tailed_f32(113, 114, (1000, 4096)))     # ~250 workgroups
    bb2 = synth.f32_to_bf16_bits(synth.normal_f32(115, (1000, 4096), sigma=0.3))    # same shape, other max
    xc = synth.heavy_tailed_f32(116, 117, (300, 1040))                              # fp32, strided view
    xa_d, xb_d, xb2_d = dev_bf16(ba), dev_bf16(bb), dev_bf16(bb2)
    xc_full = dev_f32(xc)
    xc_d = xc_full[:, :1024]
    ref = {"a": _nv_ref(OF.bf16_bits_to_f32(ba)), "b": _nv_ref(OF.bf16_bits_to_f32(bb)),
           "b2": _nv_ref(OF.bf16_bits_to_f32(bb2)), "c": _nv_ref(np.ascontiguousarray(xc[:, :1024]))}
    inputs = {"a": xa_d, "b": xb_d, "b2": xb2_d, "c": xc_d}

    # 1: one stream, 70 calls
    order = ["a", "b", "c", "b2"] * 18
    outs = [(k, L.quantize_nvfp4(inputs[k])) for k in order[:70]]
    torch.cuda.synchronize()
    for i, (k, o) in enumerate(outs):
        assert _same(o, ref[k]), f"call {i} ({k})"

    # 2: two side streams, launches interleaved, no host synchronisation
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(12):
        with torch.cuda.stream(s1):
            outs.append(("b", L.quantize_nvfp4(xb_d)))
        with torch.cuda.stream(s2):
            k = "a" if i % 2 else "c"
            outs.append((k, L.quantize_nvfp4(inputs[k])))
    torch.cuda.synchronize()
    for i, (k, o) in enumerate(outs):
        assert _same(o, ref[k]), f"side-stream call {i} ({k})"

    # 3: graph replays; the static input alternates between two tensors
    # whose maxima differ, with eager library calls between the replays
    static_in = xb_d.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.quantize_nvfp4(static_in)              # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gout = L.quantize_nvfp4(static_in)
    for i in range(6):
        k = "b2" if i % 2 else "b"
        static_in.copy_(inputs[k])
        g.replay()
        torch.cuda.synchronize()
        assert _same(gout, ref[k]), f"replay {i} ({k})"
        eager = L.quantize_nvfp4(xa_d)
        torch.cuda.synchronize()
        assert _same(eager, ref["a"]), f"eager call after replay {i}"


def test_mxfp4_e2m1_rounding_sweep():
    # blocks whose maximum is 7.5 get e = 0, so the element values themselves
    # are rounded; sweep every float32 near each decision and grid point
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 7.0]
    vals = []
    for p in pts:
        b = np.array([p], F32).view(np.int32)[0]
        vals.extend(np.arange(b - 600, b + 601, dtype=np.int32).view(F32).tolist())
    rng = np.random.default_rng(105)
    vals.extend(rng.uniform(-7.99, 7.99, 200000).astype(F32).tolist())
    vals.extend([0.0, -0.0, 1e-45, -1e-45, 1e-30])
    v = np.array(vals, F32)
    v = np.concatenate([v, -v])
    n31 = -(-len(v) // 31)
    pad = np.zeros(n31 * 31, F32)
    pad[:len(v)] = v
    blocks = np.concatenate([np.full((n31, 1), F32(7.5)), pad.reshape(n31, 31)], axis=1)
    x = blocks.reshape(-1, 32 * 8) if n31 % 8 == 0 else np.concatenate(
        [blocks, np.tile(blocks[:1], (8 - n31 % 8, 1))]).reshape(-1, 256)
    x = np.ascontiguousarray(x, F32)
    codes, scales = fp4q().quantize_mxfp4(dev_f32(x))
    c_ref, s_ref = OMX.quantize(x)
    assert np.all(s_ref == 127)
    assert_bytes_equal(host(scales), s_ref, "mx scales")
    assert_bytes_equal(host(codes), packed(c_ref), "mx codes")


def test_mxfp4_transform_small_ragged():
    x = synth.heavy_tailed_f32(106, 107, (45, 160))
    w = synth.normal_f32(108, (33, 160), 0.02)
    _, t32, u32 = OBAL.balance_scale(w, x)
    L = fp4q()
    for arr, sc in ((x, t32), (w, u32)):
        for use_t in (False, True):
            for had in (False, True):
                c, s = L.quantize_mxfp4(dev_f32(arr), dev_f32(sc) if use_t else None, had)
                y = OMX.hadamard32_scale(arr, sc if use_t else None) if had else (
                    (arr * sc[None, :]).astype(F32) if use_t else arr)
                c_ref, s_ref = OMX.quantize(y)
                assert_bytes_equal(host(s), s_ref, f"mx scales t={use_t} h={had}")
                assert_bytes_equal(host(c), packed(c_ref), f"mx codes t={use_t} h={had}")
        yh = host(L.hadamard32_scale(dev_f32(arr), dev_f32(sc)))
        assert_bytes_equal(yh.view(np.uint32), OMX.hadamard32_scale(arr, sc).view(np.uint32), "hadamard fp32")


def test_mxfp4_transform_full_size_sampled_rows():
    wl = synth.mxfp4_transform()
    xb, wb = wl.arrays["x_bf16"], wl.arrays["w_bf16"]
    xf, wf = OF.bf16_bits_to_f32(xb), OF.bf16_bits_to_f32(wb)
    _, t32, u32 = OBAL.balance_scale(wf, xf)
    L = fp4q()
    for name, b, f, sc in (("x", xb, xf, t32), ("w", wb, wf, u32)):
        rows = sample_rows(b.shape[0], seed=7)
        d = dev_bf16(b)
        c, s = L.quantize_mxfp4(d, dev_f32(sc), True)
        c, s = host(c), host(s)
        c_ref, s_ref = OMX.quantize(OMX.hadamard32_scale(f[rows], sc))
        assert_bytes_equal(s[rows], s_ref, f"{name} scales")
        assert_bytes_equal(c[rows], packed(c_ref), f"{name} codes")
        if name == "w":
            y = L.hadamard32_scale(d, dev_f32(sc))
            c2, s2 = L.quantize_mxfp4(y)
            assert_bytes_equal(host(c2), c, "standalone rotation then quantize == fused")
            assert_bytes_equal(host(s2), s, "standalone rotation then quantize == fused (scales)")


def test_balance_scale_matches_oracle():
    wl = synth.mxfp4_transform(m=256, n=512, k=512)
    xb, wb = wl.arrays["x_bf16"], wl.arrays["w_bf16"]
    t64, t32, u32 = OBAL.balance_scale(OF.bf16_bits_to_f32(wb), OF.bf16_bits_to_f32(xb))
    t, u = fp4q().balance_scale(dev_bf16(wb), dev_bf16(xb))
    t, u = host(t), host(u)
    ulp_t = np.abs(t.view(np.int32).astype(np.int64) - t32.view(np.int32))
    ulp_u = np.abs(u.view(np.int32).astype(np.int64) - u32.view(np.int32))
    assert ulp_t.max() <= 1 and ulp_u.max() <= 1
    assert np.mean(ulp_t == 0) > 0.99


def test_balance_scale_hand_worked_columns():
    # columns whose statistics are exact powers of two, zero (floor then
    # clip at both ends) or the rms floor alone: the device statistic gives
    # the written-out values bit for bit where they are exact
    import test_oracle_nvfp4_mxfp4 as TO
    w, x, want = TO._balance_columns()
    t, u = fp4q().balance_scale(dev_f32(w.astype(np.float32)), dev_f32(x.astype(np.float32)))
    t, u = host(t), host(u)
    exact = [0, 1, 2, 3, 4]
    assert np.array_equal(t[exact], want[exact].astype(np.float32)), t
    assert np.array_equal(u[exact], (1.0 / want[exact]).astype(np.float32)), u
    _, t32, u32 = OBAL.balance_scale(w, x)
    ulp = np.abs(t.view(np.int32).astype(np.int64) - t32.view(np.int32))
    assert ulp.max() <= 1, (t, t32)


def _sd_segments(ws, steps_banks=1):
    L = fp4q()
    segs, meta = [], []
    for w in ws:
        wd = dev_f32(w)
        c0, sc, ts = L.quantize_nvfp4(wd)
        rows, cols = w.shape
        codes = torch.empty((steps_banks, rows, cols // 2), dtype=torch.uint8, device=wd.device)
        res = torch.zeros((rows, cols), dtype=torch.float32, device=wd.device)
        segs.append({"w": wd, "scales": sc, "tensor_scale": ts, "residue": res, "codes": codes})
        meta.append(c0)
    return segs, meta


def test_sigma_delta_small_segments_all_steps():
    ws = [synth.normal_f32(110 + i, shp, 0.02) for i, shp in enumerate([(48, 64), (16, 128), (7, 32)])]
    ws[0][5, 16:32] = 0.0
    segs, c0 = _sd_segments(ws)
    refs = [OSD.sigma_delta_nvfp4(w, 32) for w in ws]
    L = fp4q()
    for k in range(32):
        L.sigma_delta_requant(segs, steps=1)
        for s, ref, first in zip(segs, refs, c0):
            assert_bytes_equal(host(s["codes"][0]), packed(ref["codes"][k]), f"step {k} codes")
            assert_bytes_equal(host(s["residue"]).view(np.uint32), ref["residues"][k].view(np.uint32), f"step {k} residue")
            if k == 0:
                assert_bytes_equal(host(s["codes"][0]), host(first), "step 1 == RTN")
        r = host(segs[0]["residue"])
        assert np.abs(r).max() <= 1.0


def test_sigma_delta_multi_bank_equals_single_steps():
    ws = [synth.normal_f32(120 + i, shp, 0.02) for i, shp in enumerate([(32, 96), (64, 48)])]
    segs1, _ = _sd_segments(ws)
    segsR, _ = _sd_segments(ws, steps_banks=8)
    L = fp4q()
    singles = []
    for k in range(8):
        L.sigma_delta_requant(segs1, steps=1)
        singles.append([host(s["codes"][0]).copy() for s in segs1])
    stride = max(w.shape[0] * w.shape[1] // 2 for w in ws)
    stride = -(-stride // 16) * 16
    # banks of each segment must be spaced by one common stride: allocate per segment
    for s, w in zip(segsR, ws):
        s["codes"] = torch.empty((8, stride), dtype=torch.uint8, device=s["w"].device)
    L.sigma_delta_requant(segsR, steps=8, bank_stride=stride)
    for k in range(8):
        for j, (s, w) in enumerate(zip(segsR, ws)):
            n = w.shape[0] * w.shape[1] // 2
            assert_bytes_equal(host(s["codes"][k, :n]).reshape(w.shape[0], -1), singles[k][j], f"bank {k}")
    for a, b in zip(segs1, segsR):
        assert_bytes_equal(host(a["residue"]).view(np.uint32), host(b["residue"]).view(np.uint32), "final residue")


def test_sigma_delta_looped_core_full_size_sampled_rows():
    wl = synth.looped_sigma_delta(tokens=8)
    ws = [wl.arrays[f"w{i}"] for i in range(13)]
    segs, _ = _sd_segments(ws)
    L = fp4q()
    samples = [sample_rows(w.shape[0], k=12, seed=i) for i, w in enumerate(ws)]
    refs = []
    for w, rows, s in zip(ws, samples, segs):
        st = ONV.tensor_scale_from_amax(np.abs(w).max())      # the oracle's own, over the whole weight
        assert host(s["tensor_scale"])[0] == st
        refs.append(OSD.sigma_delta_nvfp4(w[rows], 32, tensor_scale=st))
    for k in range(32):
        L.sigma_delta_requant(segs, steps=1)
        if k in (0, 1, 2, 15, 31):
            for s, ref, rows in zip(segs, refs, samples):
                assert_bytes_equal(host(s["codes"][0])[rows], packed(ref["codes"][k]), f"step {k}")
                assert_bytes_equal(host(s["residue"])[rows].view(np.uint32), ref["residues"][k].view(np.uint32), f"res {k}")


def test_sigma_delta_reverse_tail_schedule():
    # B nearest-code banks, then a fresh chain of K codes in reverse, one launch
    ws = [synth.normal_f32(130 + i, shp, 0.02) for i, shp in enumerate([(48, 64), (16, 128), (7, 32)])]
    ws[0][5, 16:32] = 0.0
    L = fp4q()
    for B, K in ((3, 5), (0, 4), (2, 1), (0, 1)):
        segs, _ = _sd_segments(ws)
        stride = -(-max(w.size // 2 for w in ws) // 16) * 16
        for s_ in segs:
            s_["codes"] = torch.empty((B + K, stride), dtype=torch.uint8, device=s_["w"].device)
            s_["residue"] = None
        print(f"reverse-tail schedule B={B} K={K}", flush=True)
        L.sigma_delta_schedule(segs, B, K, bank_stride=stride)
        for s_, w in zip(segs, ws):
            want = OSD.reverse_tail_schedule(w, B, K)
            got = host(s_["codes"])
            for b in range(B + K):
                assert_bytes_equal(got[b, :w.size // 2].reshape(w.shape[0], -1), packed(want[b]), f"B={B} K={K} bank {b}")


def test_sigma_delta_reverse_tail_looped_core_full_size():
    # the 13 linears of the looped core, 4 nearest-code + 28 tail accesses
    wl = synth.looped_sigma_delta(tokens=8)
    ws = [wl.arrays[f"w{i}"] for i in range(13)]
    segs, _ = _sd_segments(ws)
    B, K = 4, 28
    stride = -(-max(w.size // 2 for w in ws) // 16) * 16
    for s_ in segs:
        s_["codes"] = torch.empty((B + K, stride), dtype=torch.uint8, device=s_["w"].device)
        s_["residue"] = None
    print("reverse-tail schedule, looped core", flush=True)
    L = fp4q()
    L.sigma_delta_schedule(segs, B, K, bank_stride=stride)
    for i, (s_, w) in enumerate(zip(segs, ws)):
        rows = sample_rows(w.shape[0], k=6, seed=i)
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        want = OSD.reverse_tail_schedule(w[rows], B, K, tensor_scale=st)
        got = host(s_["codes"])
        for b in (0, B - 1, B, B + 7, B + K - 1):
            bank = got[b, :w.size // 2].reshape(w.shape[0], -1)[rows]
            assert_bytes_equal(bank, packed(want[b]), f"linear {i} bank {b}")


def _sr_segments(ws, steps):
    segs, _ = _sd_segments(ws)
    stride = -(-max(w.size // 2 for w in ws) // 16) * 16
    for s_ in segs:
        s_["codes"] = torch.empty((steps, stride), dtype=torch.uint8, device=s_["w"].device)
        s_["residue"] = None
    return segs, stride


def test_stochastic_rounding_small_segments_bit_exact():
    # 18 segments: two launches of the segment table, so the segment index
    # in the Philox counter must continue across them
    shapes = [(48, 64), (16, 128), (7, 32)] * 6
    ws = [synth.normal_f32(140 + i, shp, 0.02) for i, shp in enumerate(shapes)]
    ws[0][5, 16:32] = 0.0
    ws[1][2, :16] = -0.0
    segs, stride = _sr_segments(ws, 5)
    print("stochastic rounding, 18 segments x 5 accesses", flush=True)
    L = fp4q()
    L.stochastic_round_requant(segs, 5, seed=42, step0=7, bank_stride=stride)
    for i, (s_, w) in enumerate(zip(segs, ws)):
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        want = OSD.stochastic_rounding_nvfp4(w, 5, 42, step0=7, segment=i, tensor_scale=st)
        got = host(s_["codes"])
        for k in range(5):
            assert_bytes_equal(got[k, :w.size // 2].reshape(w.shape[0], -1), packed(want[k]), f"segment {i} access {k}")


def test_stochastic_rounding_looped_core_full_size():
    wl = synth.looped_sigma_delta(tokens=8)
    ws = [wl.arrays[f"w{i}"] for i in range(13)]
    R = 32
    segs, stride = _sr_segments(ws, R)
    print("stochastic rounding, looped core, 32 accesses", flush=True)
    L = fp4q()
    seed = 0x5EED_0000_002A
    L.stochastic_round_requant(segs, R, seed=seed, bank_stride=stride)
    for i, (s_, w) in enumerate(zip(segs, ws)):
        rows = sample_rows(w.shape[0], k=6, seed=i)
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        want = OSD.stochastic_rounding_nvfp4(w, R, seed, segment=i, rows=rows, tensor_scale=st)
        got = host(s_["codes"])
        for k in (0, 1, 17, R - 1):
            bank = got[k, :w.size // 2].reshape(w.shape[0], -1)[rows]
            assert_bytes_equal(bank, packed(want[k]), f"linear {i} access {k}")


def test_two_point_chain_bit_exact():
    # small segments (zero and -0 blocks, tiny values near zero) and the
    # looped core on sampled rows; banks hold accesses step0 + 1 ..
    ws = [synth.normal_f32(150 + i, shp, 0.02) for i, shp in enumerate([(24, 64), (8, 128), (7, 32)])]
    ws[0][5, 16:32] = 0.0
    ws[1][2, :16] = -0.0
    ws[1][3, 16:32] *= 1e-9                     # normalised values near zero: tiny
    ws[1][3, 16] = 0.02                         # values beside one block maximum
    L = fp4q()
    segs, stride = _sr_segments(ws, 6)
    print("two-point chain, 3 segments x 6 accesses", flush=True)
    L.two_point_requant(segs, 6, step0=3, bank_stride=stride)
    for i, (s_, w) in enumerate(zip(segs, ws)):
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        want = OSD.two_point_nvfp4(w, range(4, 10), tensor_scale=st)
        got = host(s_["codes"])
        for j in range(6):
            assert_bytes_equal(got[j, :w.size // 2].reshape(w.shape[0], -1), packed(want[4 + j]), f"segment {i} access {4 + j}")
    wl = synth.looped_sigma_delta(tokens=8)
    ws = [wl.arrays[f"w{i}"] for i in (0, 4, 12)]
    segs, stride = _sr_segments(ws, 32)
    print("two-point chain, looped-core linears x 32 accesses", flush=True)
    L.two_point_requant(segs, 32, bank_stride=stride)
    for i, (s_, w) in enumerate(zip(segs, ws)):
        rows = sample_rows(w.shape[0], k=2, seed=i)
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        want = OSD.two_point_nvfp4(w, (1, 2, 17, 32), rows=rows, tensor_scale=st)
        got = host(s_["codes"])
        for k in (1, 2, 17, 32):
            bank = got[k - 1, :w.size // 2].reshape(w.shape[0], -1)[rows]
            assert_bytes_equal(bank, packed(want[k]), f"linear {i} access {k}")
