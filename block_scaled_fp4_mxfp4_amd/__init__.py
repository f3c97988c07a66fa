"""libfp4q: block-scaled FP4 (NVFP4 / MXFP4) W4A4 linear layer and looped
Sigma-Delta re-quantization on AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libfp4q.so`` (C ABI, ``include/fp4q.h``);
``block_scaled_fp4_mxfp4_amd.fp4q`` is a thin ctypes binding over it, imported
explicitly (``from block_scaled_fp4_mxfp4_amd import fp4q``) so that input
generation (``synth``) works on hosts without the library.
"""
