"""CPU oracle for FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain definition the GPU
library is checked against.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
it shares no code, tables or constants with the HIP kernels.

Contents
  formats  -- E4M3 / E5M2 decode and the saturating round-to-nearest-even cast
              (two independent encoders: nearest-value search and binade rounding)
  quant    -- scale granularities, amax, fp32 and E8M0 scale rules, quantize,
              dequantize, delayed scaling, and the FP8 KV-cache codec
              (quantize on append, dequantize on read, static scales per
              tensor / head / channel)
  fp4      -- E2M1 (FP4) with MXFP4 (32-element UE8M0) and NVFP4 (16-element
              E4M3 microscale + fp32 tensor scale) quantize, dequantize and the
              GEMM reference
  gemm     -- exact (fp64) GEMM on the dequantized operands, |x|.|w| bound and the
              elementwise tolerance test

Precision: fp64 throughout.  Where a value is defined as an fp32 result of one
operation (the scale amax/Vmax, the scaled element x/s, the dequantized x*s),
the fp64 result is rounded once to fp32; for a single +,-,*,/ of fp32 operands
an fp64 intermediate gives the correctly rounded fp32 result (53 >= 2*24+2), so
this equals the direct fp32 operation.  The tests pin that against exact
rational arithmetic.

Every function with no pin other than the GPU would say "parity unpinned"; at
present every function here is pinned by tests under tests/test_oracle_*.py.
"""

from . import formats, quant, gemm  # noqa: F401
