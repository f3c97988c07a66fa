"""CPU oracle for block-scaled FP4 (NVFP4 / MXFP4) quantization, the block-32
Hadamard transform, first-order Sigma-Delta re-quantization and the W4A4 /
W4A16 GEMMs.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``block_scaled_fp4_mxfp4_amd`` and its HIP library) never imports, calls or
links anything here, and nothing here imports the product path: the two share
no code, tables or constants.

Design rules (each function docstring cites the passage it follows):

* plain, slow, obviously correct NumPy; no blocking, fusion or reordering
  beyond what the definition states;
* the fp32 steps that decide an integer (a code, a scale byte) are evaluated
  in IEEE binary32 with round-to-nearest-even, one operation at a time
  (NumPy never contracts a*b+c into an FMA), because that is the precision
  the formats fix (FP32 tensor scale, E4M3 / E8M0 block scales);
* everything that is not such a decision (dequantization, the GEMM, the
  balance-scale statistics) is computed in float64;
* the E2M1 rounding is the definition itself -- nearest point of the finite
  code book, ties to the even code -- evaluated by exhaustive comparison with
  the eight magnitudes, not by a threshold table.

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_*.py``.  Functions with no independent pin say
"parity unpinned" in their docstring; at present there are none.
"""

from . import formats, nvfp4, mxfp4, sigma_delta, gemm, balance  # noqa: F401
