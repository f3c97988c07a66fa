"""CPU-side checks of the C ABI: the library loads, exports every entry
point include/fp4q.h declares, and rejects invalid arguments with the
documented status codes before touching any device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")
LIB = os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "libfp4q.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def fp4q():
    if not os.path.exists(LIB):
        pytest.skip("libfp4q.so not built")
    from block_scaled_fp4_mxfp4_amd import fp4q as m
    return m


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["fp4q_quantize_nvfp4", "fp4q_quantize_mxfp4", "fp4q_hadamard32_scale",
              "fp4q_sigma_delta_requant", "fp4q_gemm_w4a4", "fp4q_gemm_w4a16", "fp4q_linear_w4a4",
              "fp4q_balance_scale", "fp4q_harmonize_nvfp4", "fp4q_hessian_accumulate",
              "fp4q_macaq_workspace_bytes", "fp4q_macaq_refine", "fp4q_sigma_delta_schedule",
              "fp4q_stochastic_round_requant", "fp4q_gemm_w4a16_grouped", "fp4q_two_point_requant",
              "fp4q_abi_version", "fp4q_status_str",
              "fp4q_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(fp4q):
    lib = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(fp4q.EXPORTED)
    assert fp4q.abi_version() == 1
    assert fp4q.lib.fp4q_status_str(2) == b"FP4Q_ERR_BAD_SHAPE"


def test_validation_happens_before_any_device_work(fp4q):
    L = fp4q.lib
    P = ctypes.c_void_p
    fake = P(0x1000)          # never dereferenced: validation fails first
    fake16 = P(0x10000)
    assert L.fp4q_quantize_nvfp4(None, 1, 4, 32, 32, fake16, fake, fake, 0, None) == 1
    assert b"NULL" in L.fp4q_last_error()
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 24, 24, fake16, fake, fake, 0, None) == 2      # cols % 16
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 16, fake16, fake, fake, 0, None) == 2      # ld < cols
    assert L.fp4q_quantize_nvfp4(P(0x1002), 1, 4, 32, 32, fake16, fake, fake, 0, None) == 3   # misaligned x
    assert L.fp4q_quantize_nvfp4(fake16, 7, 4, 32, 32, fake16, fake, fake, 0, None) == 4      # dtype
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, fake, fake, 2, None) == 5      # flag
    assert L.fp4q_quantize_nvfp4_46(fake16, 1, 4, 24, 24, fake16, fake, fake, 0, None) == 2   # cols % 16
    assert L.fp4q_quantize_nvfp4_46(None, 1, 4, 32, 32, fake16, fake, fake, 0, None) == 1
    assert L.fp4q_quantize_mxfp4(fake16, 1, 4, 48, 48, None, 0, fake16, fake, None) == 2      # cols % 32
    assert L.fp4q_quantize_mxfp4(fake16, 1, 4, 64, 64, None, 3, fake16, fake, None) == 5
    assert L.fp4q_gemm_w4a4(5, fake16, fake16, fake, fake16, fake16, fake, 4, 4, 128, fake16, 4, None) == 4
    assert L.fp4q_gemm_w4a4(0, fake16, fake16, None, fake16, fake16, fake, 4, 4, 128, fake16, 4, None) == 1
    # K must be a multiple of 32 (one MXFP4 block): 48 is refused, 96 passes
    # validation and only then meets the device check
    assert L.fp4q_gemm_w4a4(1, fake16, fake16, None, fake16, fake16, None, 4, 4, 48, fake16, 4, None) == 2
    assert L.fp4q_gemm_w4a4(1, fake16, fake16, None, fake16, fake16, None, 4, 4, 96, fake16, 4, None) == 6
    assert L.fp4q_gemm_w4a16(fake16, 96, fake16, fake16, fake, 4, 4, 80, fake16, 4, None) == 2
    assert L.fp4q_gemm_w4a16(fake16, 96, fake16, fake16, fake, 4, 4, 96, fake16, 4, None) == 6
    assert L.fp4q_linear_w4a4(fake16, 160, fake, 0, fake16, fake16, fake, 2, 8, 144, fake16, 8, None) == 2
    assert L.fp4q_linear_w4a4(fake16, 160, fake, 0, fake16, fake16, fake, 2, 8, 160, fake16, 8, None) == 6
    # a computed tensor scale uses the scales buffer for 32-bit partial
    # maxima: it must be 4-byte aligned (a given tensor scale does not need it)
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1001), P(0x2000), 0, None) == 3
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1001), P(0x2000), 1, None) == 6
    # the tensor-scale cell must not lie inside the scales (4 rows x 2 bytes)
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1000), P(0x1004), 0, None) == 5
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1000), P(0x1004), 1, None) == 5
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1002), P(0x1000), 1, None) == 5   # straddles the start
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, P(0x1000), P(0x1008), 1, None) == 6
    assert L.fp4q_gemm_w4a4(1, fake16, fake16, None, fake16, fake16, None, 4, 8, 128, fake16, 4, None) == 2
    assert L.fp4q_linear_w4a4(fake16, 128, fake, 0, fake16, fake16, fake, 17, 8, 128, fake16, 8, None) == 2
    assert L.fp4q_linear_w4a4(fake16, 8192, fake, 0, fake16, fake16, fake, 1, 8, 8192, fake16, 8, None) == 2
    assert L.fp4q_gemm_w4a16(fake16, 100, fake16, fake16, fake, 4, 4, 128, fake16, 4, None) == 2
    seg = fp4q.SdSegment(0x10000, 0x1000, 0x1000, 0x10000, 0x10000, 4, 20)
    arr = (fp4q.SdSegment * 1)(seg)
    assert L.fp4q_sigma_delta_requant(arr, 1, 1, 0, None) == 2                               # cols % 16
    assert L.fp4q_sigma_delta_requant(arr, 0, 1, 0, None) == 5
    seg2 = fp4q.SdSegment(0x10000, 0x1000, 0x1000, 0x10000, 0x10000, 4, 32)
    arr2 = (fp4q.SdSegment * 1)(seg2)
    assert L.fp4q_sigma_delta_requant(arr2, 1, 4, 32, None) == 5                             # bank stride < 64
    assert L.fp4q_balance_scale(fake16, 0, 4, 4, 4, fake16, 0, 4, 4, 1.5, fake16, fake16, None) == 5
    # empty tensors are refused (BAD_SHAPE), never launched
    assert L.fp4q_quantize_nvfp4(fake16, 1, 0, 32, 32, fake16, fake, fake, 0, None) == 2
    assert L.fp4q_quantize_nvfp4(fake16, 1, 4, 0, 0, fake16, fake, fake, 0, None) == 2
    assert L.fp4q_quantize_mxfp4(fake16, 1, 0, 64, 64, None, 1, fake16, fake, None) == 2
    assert L.fp4q_hadamard32_scale(fake16, 1, 0, 64, 64, None, fake16, 64, None) == 2
    for m, n, k in ((0, 4, 128), (4, 0, 128), (4, 4, 0)):
        assert L.fp4q_gemm_w4a4(1, fake16, fake16, None, fake16, fake16, None, m, n, k, fake16, 4, None) == 2
        assert L.fp4q_gemm_w4a16(fake16, 128, fake16, fake16, fake, m, n, k, fake16, 4, None) == 2
        assert L.fp4q_linear_w4a4(fake16, 128, fake, 0, fake16, fake16, fake, m, n, k, fake16, 8, None) == 2
    seg0 = fp4q.SdSegment(0x10000, 0x1000, 0x1000, 0x10000, 0x10000, 0, 32)
    assert L.fp4q_sigma_delta_requant((fp4q.SdSegment * 1)(seg0), 1, 1, 0, None) == 2
    # the reverse-tail schedule: residue not required; bank counts and stride checked
    segn = (fp4q.SdSegment * 1)(fp4q.SdSegment(0x10000, 0x1000, 0x1000, 0, 0x10000, 4, 32))
    assert L.fp4q_sigma_delta_schedule(segn, 1, -1, 4, 64, None) == 5
    assert L.fp4q_sigma_delta_schedule(segn, 1, 2, 0, 64, None) == 5
    assert L.fp4q_sigma_delta_schedule(segn, 1, 2, 4, 32, None) == 5                  # stride < 64
    assert L.fp4q_sigma_delta_schedule(segn, 0, 2, 4, 64, None) == 5
    assert L.fp4q_sigma_delta_schedule((fp4q.SdSegment * 1)(seg0), 1, 2, 4, 64, None) == 2
    # stochastic rounding: residue not required; steps and stride checked
    assert L.fp4q_stochastic_round_requant(segn, 1, 0, 64, 42, 0, None) == 5
    assert L.fp4q_stochastic_round_requant(segn, 1, 4, 48, 42, 0, None) == 5
    assert L.fp4q_stochastic_round_requant(segn, 65, 4, 64, 42, 0, None) == 5
    assert L.fp4q_stochastic_round_requant((fp4q.SdSegment * 1)(seg0), 1, 1, 0, 42, 0, None) == 2
    assert L.fp4q_two_point_requant(segn, 1, 0, 64, 0, None) == 5
    assert L.fp4q_two_point_requant(segn, 1, 4, 64, (1 << 24) - 3, None) == 5      # step0 + steps >= 2^24
    assert L.fp4q_two_point_requant(segn, 1, 4, 16, 0, None) == 5


def test_harmonize_validation(fp4q):
    L, M = fp4q.lib, fp4q.NvMember
    cell = ctypes.c_void_p(0x90000)

    def call(*mems, shared=cell):
        return L.fp4q_harmonize_nvfp4((M * max(len(mems), 1))(*mems), len(mems), shared, None)

    a = M(0x10000, 0x80000, 8, 64)                   # 32 scale bytes at 0x10000
    b = M(0x20000, 0x80004, 8, 64)
    assert call(a, b, shared=None) == 1
    assert call(M(0, 0x80000, 8, 64), b) == 1
    assert call() == 5                                          # n_members = 0
    assert L.fp4q_harmonize_nvfp4((M * 17)(*([a] * 17)), 17, cell, None) == 5
    assert call(M(0x10000, 0x80000, 8, 40), b) == 2             # cols % 16
    assert call(M(0x10000, 0x80000, 0, 64), b) == 2             # empty
    assert call(a, M(0x1001F, 0x80004, 8, 64)) == 5             # scale ranges overlap by one byte
    assert call(a, M(0x20000, 0x1001C, 8, 64)) == 5             # a tensor-scale cell inside a's scales
    assert call(a, b, shared=ctypes.c_void_p(0x2001D)) == 5     # shared cell straddles b's last bytes
    assert b"overlap" in L.fp4q_last_error()


def test_device_check_without_gpu(fp4q):
    import torch
    if torch.cuda.is_available():
        pytest.skip("host has a GPU")
    fake16 = ctypes.c_void_p(0x10000)
    st = fp4q.lib.fp4q_quantize_nvfp4(fake16, 1, 4, 32, 32, fake16, fake16, ctypes.c_void_p(0x20000), 0, None)
    assert st == 6


def test_macaq_validation(fp4q):
    L = fp4q.lib
    P = ctypes.c_void_p
    f16, f8 = P(0x10000), P(0x10008)
    assert L.fp4q_hessian_accumulate(None, 4, 8, 8, f16, None) == 1
    assert L.fp4q_hessian_accumulate(f16, 0, 8, 8, f16, None) == 2
    assert L.fp4q_hessian_accumulate(f16, 4, 8, 4, f16, None) == 2           # ldx < n
    assert L.fp4q_macaq_workspace_bytes(10, 64) == 8 * (32 + 64 + 640)
    assert L.fp4q_macaq_workspace_bytes(10, 16400) == -1
    ws = L.fp4q_macaq_workspace_bytes(10, 64)
    ok = dict(w=f16, m=10, n=64, ldw=64, h=f16, lam=1.0, k=128, codes=f16, scales=f16, flips=None,
              ws=f16, wsb=ws)

    def call(**kw):
        a = {**ok, **kw}
        return L.fp4q_macaq_refine(a["w"], a["m"], a["n"], a["ldw"], a["h"], a["lam"], a["k"], a["codes"],
                                   a["scales"], a["flips"], a["ws"], a["wsb"], None)

    assert call(h=None) == 1
    assert call(n=48) == 2 and call(n=16) == 2 and call(n=16416, ldw=16416) == 2
    assert call(ldw=66) == 2 and call(m=0) == 2
    assert call(w=P(0x10004)) == 3 and call(codes=f8) == 3 and call(ws=P(0x10004)) == 3
    assert call(lam=-1.0) == 5 and call(lam=float("nan")) == 5 and call(k=-1) == 5
    assert call(wsb=ws - 8) == 5
    assert b"workspace" in L.fp4q_last_error()


def test_macaq_noalloc_validation(fp4q):
    L = fp4q.lib
    P = ctypes.c_void_p
    f16, f8 = P(0x10000), P(0x10008)
    ok = dict(w=f16, m=10, n=64, ldw=64, h=f16, lam=1.0, k=128, codes=f16, scales=f16, flips=None)

    def call(**kw):
        a = {**ok, **kw}
        return L.fp4q_macaq_refine_noalloc(a["w"], a["m"], a["n"], a["ldw"], a["h"], a["lam"], a["k"],
                                           a["codes"], a["scales"], a["flips"], None)

    assert call(w=None) == 1 and call(scales=None) == 1
    assert call(n=48) == 2 and call(n=16416, ldw=16416) == 2 and call(m=0) == 2
    assert b"16384" in L.fp4q_last_error()
    assert call(w=P(0x10004)) == 3 and call(codes=f8) == 3
    assert call(lam=-1.0) == 5 and call(k=(1 << 20) + 1) == 5


def test_w4a16_grouped_validation(fp4q):
    L, P = fp4q.lib, fp4q.W4A16Problem
    f16 = 0x10000
    good = P(f16, 128, f16, f16, f16, 4, 4, 128, f16, 4)
    bad = P(f16, 100, f16, f16, f16, 4, 4, 128, f16, 4)               # lda < K
    assert L.fp4q_gemm_w4a16_grouped(None, 1, None) == 1
    assert L.fp4q_gemm_w4a16_grouped((P * 1)(good), 0, None) == 5
    assert L.fp4q_gemm_w4a16_grouped((P * 2)(good, bad), 2, None) == 2
    assert b"problem 1" in L.fp4q_last_error()
    nul = P(f16, 128, 0, f16, f16, 4, 4, 128, f16, 4)
    assert L.fp4q_gemm_w4a16_grouped((P * 2)(good, nul), 2, None) == 1
