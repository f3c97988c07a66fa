"""Exhaustive vetting of the hardware format conversions on the hot path,
through the C ABI, against the oracle's definitions (E2M1 "nearest code,
saturating", "Looped Transformer quantization" sections 2.1-2.2; the MXFP4
box of "MACaQ"; OCP E4M3 / E8M0 for the block scales).

* Encode: every float32 bit pattern with |x| < 8 (2 x 0x41000000 values:
  both signs, zeros, subnormals, every normal below 8) goes through
  fp4q_quantize_mxfp4 -- the quantizers' scaled E2M1 conversion -- with a
  7.99999952 anchor in every 32-block, so the block exponent is 0 and the
  converter sees x itself.  The expected codes come from the oracle's
  e2m1_round at the seven midpoints of the E2M1 grid and their neighbours:
  nearest-value rounding to a fixed grid is monotone in |x|, so those
  decisions fix the code of every pattern (checked against e2m1_round on a
  million random patterns as well).
* Decode: one-hot GEMMs return a dequantized operand exactly (a single
  non-zero product per output, exact in fp32), so every E2M1 code with
  every finite non-negative E4M3 byte (NVFP4) and every E8M0 byte (MXFP4)
  goes through each GEMM form's dequantization, on the A and on the B
  side, and is compared with the oracle's exact dequantized product.
"""
import numpy as np
import pytest
import torch

from oracle import formats as OF, gemm as OG
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = 0x41000000                     # patterns 0 .. P-1 are the magnitudes below 8
ANCHOR = 0x40FFFFFF                # 7.99999952: block maximum in [4, 8) -> exponent 0


def _thresholds():
    """Smallest magnitude bit pattern of each code 1..7, from the oracle."""
    mags = OF.E2M1_MAGNITUDES
    thr = []
    for i in range(7):
        mid = np.float32((mags[i] + mags[i + 1]) / 2)               # exact in float32
        b = int(mid.view(np.uint32))
        around = np.array([b - 1, b, b + 1], dtype=np.uint32).view(np.float32)
        c = OF.e2m1_round(around)
        assert c[0] == i and c[2] == i + 1, (i, c)
        thr.append(b if c[1] == i + 1 else b + 1)
    return thr


def _expected(t, thr):
    """Expected code of pattern index t (int64 CPU tensor): index t < P is
    magnitude pattern t, index t >= P its negative."""
    mag = t % P
    neg = t >= P
    code = torch.bucketize(mag, torch.tensor(thr, dtype=torch.int64), right=True)
    return (code + 8 * neg.to(torch.int64)).to(torch.uint8)


def test_threshold_model_equals_oracle_on_random_patterns():
    thr = _thresholds()
    rng = np.random.default_rng(8101)
    t = rng.integers(0, 2 * P, 1 << 20, dtype=np.int64)
    bits = (t % P) | ((t >= P).astype(np.int64) << 31)
    v = bits.astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(_expected(torch.from_numpy(t), thr).numpy(), OF.e2m1_round(v))


def test_e2m1_encode_every_fp32_pattern_below_8():
    L = fp4q()
    thr = _thresholds()
    rows, bpr = 16384, 128                       # 16384 rows x 128 blocks of 31 values + anchor
    per = rows * bpr * 31
    total = 2 * P
    anchor = torch.tensor([ANCHOR], dtype=torch.int32).view(torch.float32).item()
    buf = torch.empty((rows, bpr, 32), dtype=torch.float32, device=DEV)
    codes = torch.empty((rows, bpr * 16), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, bpr), dtype=torch.uint8, device=DEV)
    nchunk = -(-total // per)
    for c in range(nchunk):
        s = c * per
        n = min(per, total - s)
        print(f"encode chunk {c + 1}/{nchunk}: patterns {s}..{s + n - 1}", flush=True)
        t = torch.arange(s, s + per, dtype=torch.int64, device=DEV)
        bits = (t % P) + (t >= P).to(torch.int64) * (-(1 << 31))     # sign bit, as int32
        bits[n:] = 0
        buf[:, :, :31] = bits.to(torch.int32).view(torch.float32).view(rows, bpr, 31)
        buf[:, :, 31] = anchor
        del t, bits
        L.quantize_mxfp4(buf.view(rows, bpr * 32), out=(codes, scales))
        got = host(codes)
        sc = host(scales)
        assert (sc == 127).all(), "block exponent is not 0"
        got = torch.from_numpy(got)
        unpacked = torch.stack((got & 0xF, got >> 4), dim=-1).view(rows, bpr, 32)
        assert (unpacked[:, :, 31] == 7).all(), "anchor code"
        g = unpacked[:, :, :31].reshape(-1)[:n]
        want = _expected(torch.arange(s, s + n, dtype=torch.int64), thr)
        bad = torch.nonzero(g != want)
        if bad.numel():
            i = int(bad[0, 0])
            tt = s + i
            b = (tt % P) | ((tt >= P) << 31)
            raise AssertionError(f"{bad.numel()} mismatches in chunk {c}; first pattern 0x{b:08x}: "
                                 f"got {int(g[i])} want {int(want[i])}")


# ------------------------------------------------------------- decode ----

NV_BYTES = 127                     # E4M3 0x00 .. 0x7E (0x7F is NaN)
MX_BYTES = 255                     # E8M0 0 .. 254 (255 is NaN)


def _pattern(rows, K, block, nbytes):
    """codes[r][k] = (r + k) % 16, scale byte of block j = (r // 16 + j) % nbytes:
    any one column k meets all 16 x nbytes (code, byte) pairs over
    rows = 16 * nbytes."""
    r = np.arange(rows)[:, None]
    codes = ((r + np.arange(K)[None, :]) % 16).astype(np.uint8)
    scales = ((r // 16 + np.arange(K // block)[None, :]) % nbytes).astype(np.uint8)
    return codes, scales


def _pattern_wide(rows, K, block, nbytes):
    """codes[r][k] = (r + k) % 16, byte of block j = (j + 16 r) % nbytes: each
    row meets every pair once K / block >= nbytes."""
    r = np.arange(rows)[:, None]
    codes = ((r + np.arange(K)[None, :]) % 16).astype(np.uint8)
    scales = ((np.arange(K // block)[None, :] + 16 * r) % nbytes).astype(np.uint8)
    return codes, scales


def _one_hot(rows, K, block, one_byte, pos):
    codes = np.zeros((rows, K), np.uint8)
    codes[np.arange(rows), pos] = 2                                # 1.0
    scales = np.full((rows, K // block), one_byte, np.uint8)
    return codes, scales


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _check_exact(y, y_ref, what):
    y_ref32 = y_ref.astype(np.float32)
    bad = np.nonzero(~((y == y_ref32) | (np.isnan(y) & np.isnan(y_ref32))))
    if bad[0].size:
        i, j = bad[0][0], bad[1][0]
        raise AssertionError(f"{what}: {bad[0].size} of {y.size} differ; first [{i}, {j}] got {y[i, j]!r} "
                             f"want {y_ref32[i, j]!r}")


def _nv_run(L, ac, as_, bc, bs):
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    return host(L.gemm_w4a4(L.NVFP4, _dev(OF.pack_nibbles(ac)), _dev(as_), one,
                            _dev(OF.pack_nibbles(bc)), _dev(bs), one))


@pytest.mark.parametrize("M,K", [(256, 256), (100, 160), (16, 256), (4, 256), (1, 256)],
                         ids=["direct", "staged", "skinny16", "skinny4", "rows1"])
def test_nvfp4_gemm_dequant_every_code_and_e4m3_byte_b_side(M, K):
    L = fp4q()
    N = 16 * NV_BYTES
    bc, bs = _pattern(N, K, 16, NV_BYTES)
    pos = (np.arange(M) * 37) % K
    ac, as_ = _one_hot(M, K, 16, 0x38, pos)
    print(f"nvfp4 one-hot GEMM B side M={M} N={N} K={K}", flush=True)
    y = _nv_run(L, ac, as_, bc, bs)
    _check_exact(y, OG.w4a4_nvfp4(ac, as_, 1.0, bc, bs, 1.0), f"NVFP4 B side M={M} K={K}")


@pytest.mark.parametrize("M,K", [(2032, 256), (2032, 160), (16, 2048)], ids=["direct", "staged", "skinny16"])
def test_nvfp4_gemm_dequant_every_code_and_e4m3_byte_a_side(M, K):
    L = fp4q()
    ac, as_ = (_pattern(M, K, 16, NV_BYTES) if M > 16 else _pattern_wide(M, K, 16, NV_BYTES))
    N = K
    bc, bs = _one_hot(N, K, 16, 0x38, np.arange(N))
    print(f"nvfp4 one-hot GEMM A side M={M} N={N} K={K}", flush=True)
    y = _nv_run(L, ac, as_, bc, bs)
    _check_exact(y, OG.w4a4_nvfp4(ac, as_, 1.0, bc, bs, 1.0), f"NVFP4 A side M={M} K={K}")


@pytest.mark.parametrize("M,K", [(256, 256), (100, 160), (16, 256), (1, 256)],
                         ids=["direct", "staged", "m16", "m1"])
def test_w4a16_gemm_dequant_every_code_and_e4m3_byte(M, K):
    L = fp4q()
    N = 16 * NV_BYTES
    bc, bs = _pattern(N, K, 16, NV_BYTES)
    a = np.zeros((M, K), np.float32)
    a[np.arange(M), (np.arange(M) * 37) % K] = 1.0
    ab = synth.f32_to_bf16_bits(a)                                 # 1.0 and 0.0 are exact
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    print(f"w4a16 one-hot GEMM M={M} N={N} K={K}", flush=True)
    at = _dev(ab.view(np.int16)).view(torch.bfloat16)
    y = host(L.gemm_w4a16(at, _dev(OF.pack_nibbles(bc)), _dev(bs), one))
    _check_exact(y, OG.w4a16(ab, bc, bs, 1.0), f"W4A16 M={M} K={K}")
    yg = host(L.gemm_w4a16_grouped([(at, _dev(OF.pack_nibbles(bc)), _dev(bs), one)])[0])
    _check_exact(yg, OG.w4a16(ab, bc, bs, 1.0), f"W4A16 grouped M={M} K={K}")


def _mx_run(L, ac, as_, bc, bs):
    return host(L.gemm_w4a4(L.MXFP4, _dev(OF.pack_nibbles(ac)), _dev(as_), None,
                            _dev(OF.pack_nibbles(bc)), _dev(bs), None))


@pytest.mark.parametrize("M,K", [(256, 256), (100, 160), (16, 256)], ids=["direct", "staged", "m16"])
def test_mxfp4_gemm_every_code_and_e8m0_byte_b_side(M, K):
    L = fp4q()
    N = 16 * MX_BYTES
    bc, bs = _pattern(N, K, 32, MX_BYTES)
    ac, as_ = _one_hot(M, K, 32, 127, (np.arange(M) * 37) % K)
    print(f"mxfp4 one-hot GEMM B side M={M} N={N} K={K}", flush=True)
    y = _mx_run(L, ac, as_, bc, bs)
    with np.errstate(over="ignore"):
        _check_exact(y, OG.w4a4_mxfp4(ac, as_, bc, bs), f"MXFP4 B side M={M} K={K}")


@pytest.mark.parametrize("M,K", [(4080, 256), (4080, 160)], ids=["direct", "staged"])
def test_mxfp4_gemm_every_code_and_e8m0_byte_a_side(M, K):
    L = fp4q()
    ac, as_ = _pattern(M, K, 32, MX_BYTES)
    N = K
    bc, bs = _one_hot(N, K, 32, 127, np.arange(N))
    print(f"mxfp4 one-hot GEMM A side M={M} N={N} K={K}", flush=True)
    y = _mx_run(L, ac, as_, bc, bs)
    with np.errstate(over="ignore"):
        _check_exact(y, OG.w4a4_mxfp4(ac, as_, bc, bs), f"MXFP4 A side M={M} K={K}")
