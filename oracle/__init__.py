"""CPU oracle for the block-scaled FP4 codec -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  It is not part of the product: only the test
suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, tables or constants with the
HIP path under ``block_scaled_fp4_amd/``, and it never imports that package.

Modules
-------
formats   E2M1 / E4M3 / UE8M0 / bf16 element formats (decode, RTN, SR).
philox    Philox4x32-10 counter-based generator (Salmon et al., SC'11).
nvfp4     NVFP4 quantize / dequantize / error-feedback qdq.
mxfp4     MXFP4 quantize / dequantize.
fp4quant  FP4Quant group codec (RMS scale, normalized WHT, absmax scale).
fp8col    MXFP4 rows -> FP8 E4M3 columns with 4-to-1 scale alignment.

Every function cites the page and section it follows.  Where the pages leave
a step open, the reading taken is stated in the docstring and marked
"[reading]".  Pins against facts outside the oracle live in ``tests/``.

Parity status: every function here is pinned by at least one test that does
not re-type its own formula.  The nibble order inside a packed byte
(``pack_codes``), which no page fixes, is pinned to ROCm's host-side fp4x2
storage conversion (hip/hip_fp4.h), an implementation outside this package.
"""
