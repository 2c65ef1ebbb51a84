"""CPU oracle for the block-quantized matmul path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct re-statement of what the
method computes, in NumPy float64 (and exact ``fractions.Fraction`` for tiny
brute-force cases).  It exists to check the HIP kernels, never to stand in
for them: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It imports nothing from
the HIP path (``mixed_precision_block_amd``) and the HIP path imports nothing
from it; the two share only the seeded input generators in ``synthetic/``,
which hold none of the method's arithmetic.

Modules
-------
formats  BF16 / E2M1 / E4M3FN / E8M0 decode and round-to-nearest-even encode
quant    per-32 block quantization with power-of-two (E8M0) scales
gemm     dequantized fp64 products, exact rational brute force, tolerances
arc      ARCQuant augmented residual channels (selection, residual, K' GEMM)
ramp     RAMP recurrent-depth step and precision schedule
gemv     8-bit weights read as top nibble, escalation of flagged tokens
gate     entropy / margin escalation gate over low-pass logits
kvquant  FP8 per-token-head-tile-128 quantize-on-write (float32 scales)

Parity pins
-----------
Every function is pinned by ``tests/test_oracle_*.py`` against things other
than itself: values derived by hand from the format definitions
(``tests/golden/``), library routines (torch's float8_e4m3fn and bfloat16
casts, torch rms_norm/silu in float64), exact rational brute force on tiny
inputs, closed forms and invariants.  One quantity is **parity unpinned**:
the ARCQuant page's dual-stage error-bound constant (about 1.266 versus < 2
for MXFP8) has no formula on the page, so the oracle only reports the ARC vs
plain-MXFP4 error ordering and does not check that constant.
"""

from . import formats, quant, gemm, arc, ramp, gemv, gate, kvquant  # noqa: F401
