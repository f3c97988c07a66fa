"""ctypes binding of libfp4q (``include/fp4q.h``).

Argument marshalling only: every computation runs in the HIP library.  Torch
tensors provide device memory and the current stream; outputs are allocated
here with ``torch.empty`` on the input's device and returned.  If the library
is missing or fails to load, importing this module raises -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libfp4q.so not built ({LIB_PATH}); run __graft_entry__.build()")
lib = ctypes.CDLL(LIB_PATH)

F32, BF16 = 0, 1
NVFP4, MXFP4 = 0, 1
STATUS = {0: "FP4Q_OK", 1: "FP4Q_ERR_NULL_PTR", 2: "FP4Q_ERR_BAD_SHAPE", 3: "FP4Q_ERR_BAD_ALIGN",
          4: "FP4Q_ERR_BAD_DTYPE", 5: "FP4Q_ERR_BAD_ARG", 6: "FP4Q_ERR_DEVICE", 7: "FP4Q_ERR_LAUNCH"}

_p = ctypes.c_void_p
_i = ctypes.c_int
_l = ctypes.c_int64


class SdSegment(ctypes.Structure):
    _fields_ = [("w", _p), ("scales", _p), ("tensor_scale", _p), ("residue", _p),
                ("codes", _p), ("rows", _l), ("cols", _l)]


class W4A16Problem(ctypes.Structure):
    _fields_ = [("a_bf16", _p), ("lda", _l), ("b_codes", _p), ("b_scales", _p), ("b_tscale", _p),
                ("M", _l), ("N", _l), ("K", _l), ("y", _p), ("ldy", _l)]


class NvMember(ctypes.Structure):
    _fields_ = [("scales", _p), ("tensor_scale", _p), ("rows", _l), ("cols", _l)]


_SIGS = {
    "fp4q_abi_version": ([], _i),
    "fp4q_status_str": ([_i], ctypes.c_char_p),
    "fp4q_last_error": ([], ctypes.c_char_p),
    "fp4q_quantize_nvfp4": ([_p, _i, _l, _l, _l, _p, _p, _p, _i, _p], _i),
    "fp4q_quantize_nvfp4_46": ([_p, _i, _l, _l, _l, _p, _p, _p, _i, _p], _i),
    "fp4q_quantize_mxfp4": ([_p, _i, _l, _l, _l, _p, _i, _p, _p, _p], _i),
    "fp4q_hadamard32_scale": ([_p, _i, _l, _l, _l, _p, _p, _l, _p], _i),
    "fp4q_balance_scale": ([_p, _i, _l, _l, _l, _p, _i, _l, _l, ctypes.c_double, _p, _p, _p], _i),
    "fp4q_sigma_delta_requant": ([ctypes.POINTER(SdSegment), _i, _i, _l, _p], _i),
    "fp4q_sigma_delta_schedule": ([ctypes.POINTER(SdSegment), _i, _i, _i, _l, _p], _i),
    "fp4q_two_point_requant": ([ctypes.POINTER(SdSegment), _i, _i, _l, ctypes.c_uint32, _p], _i),
    "fp4q_stochastic_round_requant": ([ctypes.POINTER(SdSegment), _i, _i, _l, ctypes.c_uint64, ctypes.c_uint32,
                                       _p], _i),
    "fp4q_harmonize_nvfp4": ([ctypes.POINTER(NvMember), _i, _p, _p], _i),
    "fp4q_hessian_accumulate": ([_p, _l, _l, _l, _p, _p], _i),
    "fp4q_macaq_workspace_bytes": ([_l, _l], _l),
    "fp4q_macaq_refine": ([_p, _l, _l, _l, _p, ctypes.c_double, _i, _p, _p, _p, _p, _l, _p], _i),
    "fp4q_macaq_refine_noalloc": ([_p, _l, _l, _l, _p, ctypes.c_double, _i, _p, _p, _p, _p], _i),
    "fp4q_gemm_w4a4": ([_i, _p, _p, _p, _p, _p, _p, _l, _l, _l, _p, _l, _p], _i),
    "fp4q_gemm_w4a16": ([_p, _l, _p, _p, _p, _l, _l, _l, _p, _l, _p], _i),
    "fp4q_gemm_w4a16_grouped": ([ctypes.POINTER(W4A16Problem), _i, _p], _i),
    "fp4q_linear_w4a4": ([_p, _l, _p, _i, _p, _p, _p, _l, _l, _l, _p, _l, _p], _i),
}
for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTED = tuple(_SIGS)


class Fp4qError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = lib.fp4q_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp4qError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows_cols_ld(x: torch.Tensor) -> Tuple[int, int, int]:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along the last axis")
    return x.shape[0], x.shape[1], x.stride(0)


def abi_version() -> int:
    return lib.fp4q_abi_version()


# ---------------------------------------------------------------- quant ----

def quantize_nvfp4(x: torch.Tensor, tensor_scale: Optional[torch.Tensor] = None,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                   rule: str = "6"):
    """NVFP4-quantize ``x`` (fp32 or bf16 [rows, cols]).  Returns
    (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], tensor_scale
    fp32 [1]).  With ``tensor_scale`` given (fp32 [1] device tensor) it is
    used as s_t; otherwise s_t = max|x| / 1536 is computed on the device.
    ``rule="4/6"`` selects the 4/6 block scales (fp4q_quantize_nvfp4_46)."""
    if rule not in ("6", "4/6"):
        raise ValueError(f"rule must be '6' or '4/6', not {rule!r}")
    rows, cols, ld = _rows_cols_ld(x)
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        codes, scales, ts = out
    is_input = 0
    if tensor_scale is not None:
        if ts.data_ptr() != tensor_scale.data_ptr():
            ts.copy_(tensor_scale)
        is_input = 1
    fn = lib.fp4q_quantize_nvfp4 if rule == "6" else lib.fp4q_quantize_nvfp4_46
    _check(fn(_ptr(x), _dtype_code(x), rows, cols, ld, _ptr(codes), _ptr(scales),
              _ptr(ts), is_input, _stream(dev)), "quantize_nvfp4")
    return codes, scales, ts


def quantize_mxfp4(x: torch.Tensor, chan_scale: Optional[torch.Tensor] = None, hadamard: bool = False,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """MXFP4-quantize ``x`` after the optional balance scale and block-32
    Hadamard rotation.  Returns (codes [rows, cols/2], scales [rows, cols/32])."""
    rows, cols, ld = _rows_cols_ld(x)
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    else:
        codes, scales = out
    _check(lib.fp4q_quantize_mxfp4(_ptr(x), _dtype_code(x), rows, cols, ld, _ptr(chan_scale), int(hadamard),
                                   _ptr(codes), _ptr(scales), _stream(dev)), "quantize_mxfp4")
    return codes, scales


def hadamard32_scale(x: torch.Tensor, chan_scale: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    rows, cols, ld = _rows_cols_ld(x)
    y = torch.empty((rows, cols), dtype=torch.float32, device=x.device) if out is None else out
    _check(lib.fp4q_hadamard32_scale(_ptr(x), _dtype_code(x), rows, cols, ld, _ptr(chan_scale), _ptr(y),
                                     y.stride(0), _stream(x.device)), "hadamard32_scale")
    return y


def balance_scale(w: torch.Tensor, x: torch.Tensor, alpha: float = 0.75):
    """Per-channel balance scale from weights w [N, K] and calibration
    activations x [M, K].  Returns (t fp32 [K], u = 1/t fp32 [K])."""
    n, k, ldw = _rows_cols_ld(w)
    m, k2, ldx = _rows_cols_ld(x)
    if k != k2:
        raise ValueError("w and x must have the same number of columns")
    t = torch.empty(k, dtype=torch.float32, device=w.device)
    u = torch.empty(k, dtype=torch.float32, device=w.device)
    _check(lib.fp4q_balance_scale(_ptr(w), _dtype_code(w), n, k, ldw, _ptr(x), _dtype_code(x), m, ldx,
                                  float(alpha), _ptr(t), _ptr(u), _stream(w.device)), "balance_scale")
    return t, u


def sigma_delta_requant(segments: Sequence[dict], steps: int = 1, bank_stride: int = 0) -> None:
    """Run ``steps`` Sigma-Delta re-quantization steps over the given weights
    in one launch.  Each segment is a dict with device tensors ``w`` (fp32
    [rows, cols]), ``scales`` (E4M3 [rows, cols/16]), ``tensor_scale`` (fp32
    [1]), ``residue`` (fp32 [rows, cols], in/out) and ``codes`` (uint8, bank
    0 at its start)."""
    arr = (SdSegment * len(segments))()
    dev = None
    for i, s in enumerate(segments):
        w = s["w"]
        dev = w.device
        arr[i] = SdSegment(w.data_ptr(), s["scales"].data_ptr(), s["tensor_scale"].data_ptr(),
                           s["residue"].data_ptr(), s["codes"].data_ptr(), w.shape[0], w.shape[1])
    _check(lib.fp4q_sigma_delta_requant(arr, len(segments), int(steps), int(bank_stride), _stream(dev)),
           "sigma_delta_requant")


def harmonize_nvfp4(scales: Sequence[torch.Tensor], tensor_scales: Sequence[torch.Tensor],
                    shared: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Give the members of a fused NVFP4 GEMM one shared tensor scale.  Each
    member is its E4M3 block scales (uint8 [rows, cols/16], rewritten in
    place) and its fp32 [1] tensor scale (overwritten with the shared one).
    Returns the shared scale (fp32 [1]; ``shared`` if given)."""
    if len(scales) != len(tensor_scales):
        raise ValueError("one tensor scale per member")
    arr = (NvMember * len(scales))()
    for i, (sb, ts) in enumerate(zip(scales, tensor_scales)):
        if sb.dtype != torch.uint8 or sb.dim() != 2 or not sb.is_contiguous():
            raise ValueError("member scales must be contiguous uint8 [rows, cols/16]")
        arr[i] = NvMember(sb.data_ptr(), ts.data_ptr(), sb.shape[0], sb.shape[1] * 16)
    dev = scales[0].device if len(scales) else torch.device("cuda")
    out = torch.empty(1, dtype=torch.float32, device=dev) if shared is None else shared
    _check(lib.fp4q_harmonize_nvfp4(arr, len(scales), _ptr(out), _stream(dev)), "harmonize_nvfp4")
    return out


def hessian_accumulate(x: torch.Tensor, h: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h += x^T x (float64 [n, n]) for fp32 calibration rows x [T, n];
    a zero h is allocated when none is given."""
    if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be fp32 [T, n] with unit column stride")
    n = x.shape[1]
    if h is None:
        h = torch.zeros((n, n), dtype=torch.float64, device=x.device)
    _check(lib.fp4q_hessian_accumulate(_ptr(x), x.shape[0], n, x.stride(0), _ptr(h), _stream(x.device)),
           "hessian_accumulate")
    return h


def macaq_refine(w: torch.Tensor, h: torch.Tensor, lam: float = 1.0, k_iters: int = 128,
                 workspace: Optional[torch.Tensor] = None):
    """Exponent screen + Flip-Refinement of the fp32 transformed weight w
    [m, n] under the calibration Hessian h [n, n] (float64).  Returns
    (codes uint8 [m, n/2], scales uint8 [m, n/32], flips int32 [m])."""
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be fp32 [m, n] with unit column stride")
    if h.dtype != torch.float64 or not h.is_contiguous():
        raise ValueError("h must be contiguous float64 [n, n]")
    m, n = w.shape
    codes = torch.empty((m, n // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((m, n // 32), dtype=torch.uint8, device=w.device)
    flips = torch.empty(m, dtype=torch.int32, device=w.device)
    need = lib.fp4q_macaq_workspace_bytes(m, n)
    if workspace is None:
        workspace = torch.empty(max(need, 8) // 8, dtype=torch.float64, device=w.device)
    _check(lib.fp4q_macaq_refine(_ptr(w), m, n, w.stride(0), _ptr(h), float(lam), int(k_iters), _ptr(codes),
                                 _ptr(scales), _ptr(flips), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(w.device)), "macaq_refine")
    return codes, scales, flips


def macaq_refine_noalloc(w: torch.Tensor, h: torch.Tensor, lam: float = 1.0, k_iters: int = 128,
                         out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """macaq_refine with the library's static per-device workspace: no
    device allocation when the outputs (codes, scales, flips) are passed in
    `out`.  Calls that overlap on one device race on that workspace."""
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be fp32 [m, n] with unit column stride")
    if h.dtype != torch.float64 or not h.is_contiguous():
        raise ValueError("h must be contiguous float64 [n, n]")
    m, n = w.shape
    if out is None:
        out = (torch.empty((m, n // 2), dtype=torch.uint8, device=w.device),
               torch.empty((m, n // 32), dtype=torch.uint8, device=w.device),
               torch.empty(m, dtype=torch.int32, device=w.device))
    codes, scales, flips = out
    if (codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or flips.dtype != torch.int32
            or not (codes.is_contiguous() and scales.is_contiguous() and flips.is_contiguous())
            or codes.shape != (m, n // 2) or scales.shape != (m, n // 32) or flips.shape != (m,)):
        raise ValueError("out must be contiguous (uint8 [m, n/2], uint8 [m, n/32], int32 [m])")
    _check(lib.fp4q_macaq_refine_noalloc(_ptr(w), m, n, w.stride(0), _ptr(h), float(lam), int(k_iters),
                                         _ptr(codes), _ptr(scales), _ptr(flips), _stream(w.device)),
           "macaq_refine_noalloc")
    return codes, scales, flips


def sigma_delta_schedule(segments: Sequence[dict], n_rtn: int, n_tail: int, bank_stride: int = 0) -> None:
    """Write n_rtn + n_tail code banks per weight with the reverse-order
    tail (n_rtn nearest-code banks, then a fresh chain of n_tail codes in
    reverse).  Segments as for :func:`sigma_delta_requant`; ``residue`` is
    not used."""
    arr = (SdSegment * len(segments))()
    dev = None
    for i, s in enumerate(segments):
        w = s["w"]
        dev = w.device
        res = s.get("residue")
        arr[i] = SdSegment(w.data_ptr(), s["scales"].data_ptr(), s["tensor_scale"].data_ptr(),
                           0 if res is None else res.data_ptr(), s["codes"].data_ptr(), w.shape[0], w.shape[1])
    _check(lib.fp4q_sigma_delta_schedule(arr, len(segments), int(n_rtn), int(n_tail), int(bank_stride),
                                         _stream(dev)), "sigma_delta_schedule")


def stochastic_round_requant(segments: Sequence[dict], steps: int, seed: int, step0: int = 0,
                             bank_stride: int = 0) -> None:
    """Write ``steps`` stochastic-rounding code banks per weight (Philox
    words keyed by ``seed``, accesses step0 .. step0 + steps - 1).
    Segments as for :func:`sigma_delta_requant`; ``residue`` is not used."""
    arr = (SdSegment * len(segments))()
    dev = None
    for i, s in enumerate(segments):
        w = s["w"]
        dev = w.device
        arr[i] = SdSegment(w.data_ptr(), s["scales"].data_ptr(), s["tensor_scale"].data_ptr(), 0,
                           s["codes"].data_ptr(), w.shape[0], w.shape[1])
    _check(lib.fp4q_stochastic_round_requant(arr, len(segments), int(steps), int(bank_stride),
                                             int(seed) & ((1 << 64) - 1), int(step0) & 0xFFFFFFFF, _stream(dev)),
           "stochastic_round_requant")


def two_point_requant(segments: Sequence[dict], steps: int, step0: int = 0, bank_stride: int = 0) -> None:
    """Write ``steps`` banks of the stateless two-point chain (accesses
    step0 + 1 .. step0 + steps).  Segments as for
    :func:`sigma_delta_requant`; ``residue`` is not used."""
    arr = (SdSegment * len(segments))()
    dev = None
    for i, s in enumerate(segments):
        w = s["w"]
        dev = w.device
        arr[i] = SdSegment(w.data_ptr(), s["scales"].data_ptr(), s["tensor_scale"].data_ptr(), 0,
                           s["codes"].data_ptr(), w.shape[0], w.shape[1])
    _check(lib.fp4q_two_point_requant(arr, len(segments), int(steps), int(bank_stride), int(step0) & 0xFFFFFFFF,
                                      _stream(dev)), "two_point_requant")


# ----------------------------------------------------------------- GEMM ----

def gemm_w4a4(fmt: int, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, N, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B disagree on K")
    y = torch.empty((M, N), dtype=torch.float32, device=a_codes.device) if out is None else out
    _check(lib.fp4q_gemm_w4a4(int(fmt), _ptr(a_codes), _ptr(a_scales), _ptr(a_ts), _ptr(b_codes),
                              _ptr(b_scales), _ptr(b_ts), M, N, K, _ptr(y), y.stride(0),
                              _stream(a_codes.device)), "gemm_w4a4")
    return y


def gemm_w4a16(a: torch.Tensor, b_codes, b_scales, b_ts, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K, lda = _rows_cols_ld(a)
    N = b_codes.shape[0]
    if a.dtype != torch.bfloat16 or b_codes.shape[1] * 2 != K:
        raise ValueError("a must be bf16 [M, K] matching B")
    y = torch.empty((M, N), dtype=torch.float32, device=a.device) if out is None else out
    _check(lib.fp4q_gemm_w4a16(_ptr(a), lda, _ptr(b_codes), _ptr(b_scales), _ptr(b_ts), M, N, K, _ptr(y),
                               y.stride(0), _stream(a.device)), "gemm_w4a16")
    return y


def gemm_w4a16_grouped(problems: Sequence[tuple]) -> List[torch.Tensor]:
    """Several W4A16 GEMMs in as few launches as possible.  Each problem is
    (a bf16 [M, K], b_codes, b_scales, b_ts) or with a fifth element, the
    fp32 output; returns the outputs."""
    arr = (W4A16Problem * len(problems))()
    outs = []
    dev = None
    for i, pr in enumerate(problems):
        a, bc, bs, bt = pr[:4]
        M, K, lda = _rows_cols_ld(a)
        N = bc.shape[0]
        if a.dtype != torch.bfloat16 or bc.shape[1] * 2 != K:
            raise ValueError(f"problem {i}: a must be bf16 [M, K] matching B")
        y = pr[4] if len(pr) > 4 and pr[4] is not None else torch.empty((M, N), dtype=torch.float32, device=a.device)
        arr[i] = W4A16Problem(a.data_ptr(), lda, bc.data_ptr(), bs.data_ptr(), bt.data_ptr(), M, N, K, y.data_ptr(),
                              y.stride(0))
        outs.append(y)
        dev = a.device
    _check(lib.fp4q_gemm_w4a16_grouped(arr, len(problems), _stream(dev)), "gemm_w4a16_grouped")
    return outs


def linear_w4a4(a: torch.Tensor, b_codes, b_scales, b_ts, a_tscale: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, a_ts_out: Optional[torch.Tensor] = None):
    """Fused decode linear: NVFP4-quantize bf16 ``a`` [M <= 16, K] and multiply
    by the NVFP4 weight.  Returns (y fp32 [M, N], a tensor scale fp32 [1])."""
    M, K, lda = _rows_cols_ld(a)
    N = b_codes.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=a.device) if out is None else out
    ts = torch.empty(1, dtype=torch.float32, device=a.device) if a_ts_out is None else a_ts_out
    is_input = 0
    if a_tscale is not None:
        if ts.data_ptr() != a_tscale.data_ptr():
            ts.copy_(a_tscale)
        is_input = 1
    _check(lib.fp4q_linear_w4a4(_ptr(a), lda, _ptr(ts), is_input, _ptr(b_codes), _ptr(b_scales), _ptr(b_ts),
                                M, N, K, _ptr(y), y.stride(0), _stream(a.device)), "linear_w4a4")
    return y, ts
