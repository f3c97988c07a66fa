"""The no-allocation form of the MACaQ refinement (fp4q_macaq_refine_noalloc,
workspace in the library's static per-device array) against the workspace
form (fp4q_macaq_refine), through the C ABI: codes, scales and flip counts
must be the same bytes.  Rows pass through the static workspace in chunks
of (2^21 - 32 - n) // n rows, so the shapes below cover one chunk, two
chunks with a ragged second one, and a call after a larger one (the array
keeps the earlier call's contents)."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, host, assert_bytes_equal

pytestmark = pytest.mark.gpu


def _chunk_rows(n):
    return (2 ** 21 - 32 - ((n + 31) // 32) * 32) // n


def _hessian(seed, t, n):
    x = synth.normal_f32(seed, (t, n))
    x[:, 1:] = (0.8 * x[:, :-1] + 0.6 * x[:, 1:]).astype(np.float32)
    return fp4q().hessian_accumulate(dev_f32(x))


def _compare(w, h, lam, k_iters, what):
    L = fp4q()
    m, n = w.shape
    print(f"{what}: macaq refine {m} x {n} (ldw {w.stride(0)}), K={k_iters}, "
          f"{-(-m // _chunk_rows(n))} chunk(s)", flush=True)
    want = [host(t) for t in L.macaq_refine(w, h, lam, k_iters)]
    # outputs prefilled with junk, so an unwritten byte shows
    out = (torch.full((m, n // 2), 0xA5, dtype=torch.uint8, device=w.device),
           torch.full((m, n // 32), 0x5A, dtype=torch.uint8, device=w.device),
           torch.full((m,), -7, dtype=torch.int32, device=w.device))
    got = [host(t) for t in L.macaq_refine_noalloc(w, h, lam, k_iters, out=out)]
    assert_bytes_equal(got[1], want[1], f"{what}: scales")
    assert_bytes_equal(got[0], want[0], f"{what}: codes")
    np.testing.assert_array_equal(got[2], want[2])
    return got


def test_noalloc_two_calls_second_smaller():
    n = 4096
    m = 600                                   # chunks of 510 and 90 rows
    assert _chunk_rows(n) == 510 and m > _chunk_rows(n)
    w = dev_f32(synth.heavy_tailed_f32(7101, 7102, (m, n)))
    codes, scales, flips = _compare(w, _hessian(7103, 256, n), 1.0, 128, "first call")
    assert flips.max() > 0
    # smaller, strided (ldw = 288), one chunk; the static array still holds
    # the first call's ridge, diagonal and gradient
    wide = dev_f32(synth.heavy_tailed_f32(7104, 7105, (70, 288)))
    _, _, flips2 = _compare(wide[:, :256], _hessian(7106, 96, 256), 0.25, 128, "second call")
    assert flips2.max() > 0


def test_noalloc_widest_rows_and_screen_only():
    n = 16384
    m = 130                                   # chunks of 126 and 4 rows
    assert _chunk_rows(n) == 126
    w = dev_f32(synth.heavy_tailed_f32(7201, 7202, (m, n)))
    _compare(w, _hessian(7203, 64, n), 1.0, 16, "n = 16384")
    w = dev_f32(synth.heavy_tailed_f32(7204, 7205, (40, 512)))
    _, _, flips = _compare(w, _hessian(7206, 64, 512), 1.0, 0, "k_iters = 0")
    assert (flips == 0).all()


def test_noalloc_rejects_bad_arguments():
    L = fp4q()
    w = torch.zeros((4, 16416), dtype=torch.float32, device="cuda:0")
    h = torch.zeros((1, 1), dtype=torch.float64, device="cuda:0")
    out = (torch.empty((4, 16416 // 2), dtype=torch.uint8, device="cuda:0"),
           torch.empty((4, 16416 // 32), dtype=torch.uint8, device="cuda:0"),
           torch.empty(4, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(RuntimeError, match="n <= 16384"):
        L.macaq_refine_noalloc(w, h, 1.0, 4, out=out)
