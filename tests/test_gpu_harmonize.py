"""GPU parity of the fused-member scale harmonization (one shared NVFP4
tensor scale for the members of a fused GEMM; "Why Gated DeltaNet Survives
4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM",
fused-GEMM global-scale box and pipeline step (2)) against the oracle,
through the C ABI: every block-scale byte and every scale cell must be
bit-identical, bytes around the members untouched; the fused GEMM probe
meets the GEMM bar."""
import numpy as np
import pytest
import torch

from oracle import nvfp4 as ONV, gemm as OG
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, host, assert_bytes_equal, DEV

pytestmark = pytest.mark.gpu
F32 = np.float32


def _run(member_bytes, member_ts, offsets, seed):
    """Place each member's scale bytes at the given byte offset of one
    device buffer (guard bytes between them), harmonize on the GPU and
    compare buffer and cells with the oracle."""
    L = fp4q()
    total = max(o + m.size for o, m in zip(offsets, member_bytes)) + 64
    buf_h = synth.uint8_bytes(seed, (total,))
    for o, m in zip(offsets, member_bytes):
        buf_h[o:o + m.size] = m.ravel()
    buf = torch.from_numpy(buf_h.copy()).to(DEV)
    cells = dev_f32(np.array(member_ts, F32))
    views = [buf[o:o + m.size].view(m.shape) for o, m in zip(offsets, member_bytes)]
    print(f"harmonize: {len(views)} members, sizes {[m.size for m in member_bytes]}, offsets {offsets}", flush=True)
    shared = L.harmonize_nvfp4(views, [cells[i:i + 1] for i in range(len(views))])
    want, st = ONV.harmonize(member_bytes, member_ts)
    want_buf = buf_h.copy()
    for o, w in zip(offsets, want):
        want_buf[o:o + w.size] = w.ravel()
    assert_bytes_equal(host(buf), want_buf, "harmonized scale buffer")
    assert host(shared)[0] == st
    np.testing.assert_array_equal(host(cells), np.full(len(views), st, F32))
    return buf, cells, want_buf, st


def test_harmonize_ragged_misaligned_members():
    # 1, 15, 259, 20520 and 65536 scale bytes; every alignment class; all
    # 256 byte values (invalid ones included); one member at the maximum
    shapes = [(1, 16), (3, 80), (7, 16 * 37), (513, 16 * 40), (64, 16 * 1024)]
    members = [synth.uint8_bytes(400 + i, (r, c // 16)) for i, (r, c) in enumerate(shapes)]
    ts = [F32(0.37), F32(0.0123), F32(0.5), F32(0.5 / 2.81), F32(0.2)]
    offsets, o = [], 0
    for i, m in enumerate(members):
        o += (i * 7 + 3) % 16 + 32                     # misaligned starts, guard gaps
        offsets.append(o)
        o += m.size
    buf, cells, want_buf, st = _run(members, ts, offsets, 410)
    # a second call sees equal scales everywhere: the identity
    L = fp4q()
    views = [buf[o:o + m.size].view(m.shape) for o, m in zip(offsets, members)]
    shared = L.harmonize_nvfp4(views, [cells[i:i + 1] for i in range(len(views))])
    assert_bytes_equal(host(buf), want_buf, "second call")
    assert host(shared)[0] == st


def test_harmonize_aligned_single_equal_and_zero_members():
    a = synth.uint8_bytes(420, (256, 64), 0, 0x7F)
    b = synth.uint8_bytes(421, (96, 64), 0, 0x7F)
    _run([a, b], [F32(1.0 / 1.82), F32(1.0)], [0, 256 * 64], 422)           # aligned, ratio 1.82
    _run([a], [F32(0.3)], [16], 423)                                         # one member: identity
    _run([a, b], [F32(0.25), F32(0.25)], [0, 16384 + 48], 424)               # equal scales: identity
    _run([a, b], [F32(0.0), F32(0.0)], [5, 16384 + 64], 425)                 # all zero: identity, s_t = 0
    _run([a, b], [F32(0.0), F32(0.7)], [0, 16384], 426)                      # a zero member: scales -> 0


def test_harmonize_fused_projection_full_size():
    # a fused projection the size of a 5120-wide hidden layer: members of
    # 10240 and 5120 output rows (qkv and z), member scales 1.82x apart, and
    # a 48+48-row pair (b and a) at the worst reported ratio 2.81x
    big = [synth.uint8_bytes(430, (10240, 320), 0, 0x7F), synth.uint8_bytes(431, (5120, 320), 0, 0x7F)]
    _run(big, [F32(0.0021), F32(0.0021 * 1.82)], [0, 10240 * 320], 432)
    small = [synth.uint8_bytes(433, (48, 320), 0, 0x7F), synth.uint8_bytes(434, (48, 320), 0, 0x7F)]
    _run(small, [F32(0.011 * 2.81), F32(0.011)], [0, 48 * 320], 435)


def test_harmonized_fused_gemm_probe():
    # quantize two members separately, harmonize, run ONE fused GEMM over
    # the concatenated weights: parity with the oracle's fused product, and
    # close to the members' own GEMMs (the naive fusion is not)
    L = fp4q()
    x = synth.heavy_tailed_f32(440, 441, (96, 1024))
    w1 = synth.normal_f32(442, (256, 1024), 0.02)
    w2 = synth.normal_f32(443, (128, 1024), 0.02 / 2.75)
    ac, as_, at = L.quantize_nvfp4(dev_f32(x))
    c1, s1, t1 = L.quantize_nvfp4(dev_f32(w1))
    c2, s2, t2 = L.quantize_nvfp4(dev_f32(w2))
    sep = torch.cat([L.gemm_w4a4(L.NVFP4, ac, as_, at, c1, s1, t1), L.gemm_w4a4(L.NVFP4, ac, as_, at, c2, s2, t2)], 1)
    cw = torch.cat([c1, c2])
    naive = L.gemm_w4a4(L.NVFP4, ac, as_, at, cw, torch.cat([s1, s2]), torch.maximum(t1, t2))
    sw = torch.cat([s1, s2])                                  # harmonize the concatenated scales in place
    shared = L.harmonize_nvfp4([sw[:256], sw[256:]], [t1, t2])
    fused = host(L.gemm_w4a4(L.NVFP4, ac, as_, at, cw, sw, shared))
    sep, naive = host(sep), host(naive)
    cx, sx, tx = ONV.quantize(x)
    o1, q1, u1 = ONV.quantize(w1)
    o2, q2, u2 = ONV.quantize(w2)
    (h1, h2), st = ONV.harmonize([q1, q2], [u1, u2])
    assert host(shared)[0] == st
    assert_bytes_equal(host(sw), np.concatenate([h1, h2]), "harmonized scales")
    ref = OG.w4a4_nvfp4(cx, sx, tx, np.concatenate([o1, o2]), np.concatenate([h1, h2]), st)
    whole, row, _ = OG.rel_err(fused, ref)
    assert whole <= 1e-3 and row <= 1e-3, (whole, row)
    err_fused = OG.rel_err(fused, sep)[0]
    err_naive = OG.rel_err(naive, sep)[0]
    print(f"fused vs separate {err_fused:.4f}, naive vs separate {err_naive:.4f}")
    assert err_fused < 0.03 and err_naive > 0.3
