"""Pins for the oracle's element and scale formats (CPU only).

Each test ties ``oracle.formats`` to something other than itself: a library
routine (torch's float8 dtypes, scipy), a hand-derived golden table, the
facts the pages state (16 codes / 15 values, end points +-6, gap d = 2), or
an exact brute force in rational arithmetic.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_code_book_facts():
    # loopquant page, section 0.2: 16 codes, +0 and -0 coincide -> 15 values
    vals = F.E2M1_VALUES
    assert len(vals) == 16
    assert len(set(vals.tolist())) == 15
    # section 2.2: end points [-6, 6], largest neighbour gap d = 2
    pos = sorted(set(abs(v) for v in vals.tolist()))
    assert pos == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert min(vals) == -6.0 and max(vals) == 6.0
    full = sorted(set(vals.tolist()))
    assert max(np.diff(full)) == 2.0
    # sign bit is bit 3: code c and c|8 are negatives of each other
    for c in range(8):
        assert vals[c | 8] == -vals[c]


def test_e2m1_decode_matches_torch_float4_bits():
    # torch's float4_e2m1fn_x2 has no arithmetic, but the OCP layout can be
    # checked against the E4M3 library conversion: every E2M1 value is
    # exactly representable in E4M3, and the E2M1 -> E4M3 bit mapping is
    # sign | (e + 6) << 3 | m << 2 for normal codes.
    for c in range(16):
        v = F.E2M1_VALUES[c]
        t = torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn)
        assert float(t.float()) == v
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e > 0:
            b = int(t.view(torch.uint8))
            assert b == (s << 7) | ((e + 6) << 3) | (m << 2)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def test_e2m1_round_golden_table():
    rows = _read_golden("e2m1_round.txt")
    v = np.array([np.float32(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    got = F.e2m1_round(v)
    assert np.array_equal(got, want), list(zip(v, got, want))
    assert np.array_equal(F.e2m1_decode(got), [float(r[2]) for r in rows])


def _nearest_fraction(v: Fraction):
    """Independent brute force: sort all 8 magnitudes by (exact distance,
    mantissa bit) and take the first."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    a = abs(v)
    return min(range(8), key=lambda i: (abs(a - mags[i]), i & 1))


def test_e2m1_round_all_bf16_patterns_brute_force():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    got = F.e2m1_round(f)
    # exact rational brute force on a deterministic subsample plus every value
    # within [-8, 8] (where all the decision points are)
    near = f[np.abs(f) <= 8]
    far = f[np.abs(f) > 8][::97]
    for arr in (near, far):
        g = F.e2m1_round(arr)
        for x, c in zip(arr.tolist(), g.tolist()):
            want = _nearest_fraction(Fraction(x))
            assert c & 7 == want, (x, c)
            assert (c >> 3) == (1 if np.signbit(np.float32(x)) else 0)
    assert got.shape == f.shape


def test_e2m1_round_near_midpoints_fp32():
    # every float32 within 4 ulp of each decision midpoint and of each grid point
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = []
    for p in pts:
        b = np.array([p], np.float32).view(np.int32)[0]
        for d in range(-4, 5):
            vals.append(np.array([b + d], np.int32).view(np.float32)[0])
    vals = np.array(vals + [-v for v in vals], np.float32)
    got = F.e2m1_round(vals)
    for x, c in zip(vals.tolist(), got.tolist()):
        assert c & 7 == _nearest_fraction(Fraction(x)), x


def test_e4m3_table_matches_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = F.E4M3_VALUES
    nan_t = np.isnan(b)
    assert np.array_equal(nan_t, np.isnan(ours))
    assert np.array_equal(b[~nan_t], ours[~nan_t])
    assert F.E4M3_VALUES[0x7E] == 448.0


def test_e4m3_ceil_brute_force():
    table = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    rng = np.random.default_rng(7)
    ys = np.concatenate([
        table, np.nextafter(table, np.inf), np.nextafter(table[1:], 0),
        rng.uniform(0, 500, 2000), np.exp(rng.uniform(-25, 7, 2000)), [0.0, 448.0, 449.0, 1e6]])
    got = F.e4m3_ceil(ys)
    for y, g in zip(ys, got):
        ge = np.nonzero(table >= y)[0]
        want = ge[0] if len(ge) else 126
        assert g == want, (y, g, want)


def test_e8m0_matches_torch():
    b = torch.arange(255, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().double().numpy()
    ours = F.e8m0_decode(np.arange(255))
    assert np.array_equal(b, ours)


def test_floor_log2_exact():
    rng = np.random.default_rng(3)
    bits = rng.integers(1, 0x7F800000, size=5000, dtype=np.int64).astype(np.uint32)
    a = bits.view(np.float32)
    got = F.floor_log2_f32(a)
    for x, e in zip(a.tolist(), got.tolist()):
        fx = Fraction(x)
        assert Fraction(2) ** e <= fx < Fraction(2) ** (e + 1)


def test_nibble_packing_roundtrip_and_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0x8]], np.uint8)
    p = F.pack_nibbles(codes)
    assert p.tolist() == [[0x21, 0x43, 0x8F]]
    assert np.array_equal(F.unpack_nibbles(p), codes)


def test_bf16_widening():
    x = torch.randn(1000, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_bits_to_f32(bits), x.float().numpy())
