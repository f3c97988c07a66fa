"""libfp4q: block-scaled FP4 (NVFP4 / MXFP4) W4A4 linear layer and looped
Sigma-Delta re-quantization on AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libfp4q.so`` (C ABI, ``include/fp4q.h``);
``block_scaled_fp4_mxfp4_amd.fp4q`` is a thin ctypes binding over it.  The
binding is loaded lazily so that input generation (``synth``) can be used on
hosts without the library.
"""

__all__ = ["fp4q", "synth"]


def __getattr__(name):
    if name == "fp4q":
        from . import fp4q as _m
        return _m
    raise AttributeError(name)
