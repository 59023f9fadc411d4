"""CPU oracle for FP8 block-scaled GEMM with fine-grained scaling, and its quantizer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import or run anything in
this package.  The GPU library never calls it, and it shares no code,
constants or tables with the GPU path.

Modules:

* ``e4m3``  -- OCP E4M3 decode table and ties-to-even encode.
* ``bf16``  -- float64 -> bf16, round-to-nearest-even, in one step.
* ``quant`` -- per-token (1x128) and per-block (128x128) quantizers, with
  fp32 or power-of-two (UE8M0-style) scales.
* ``gemm``  -- dense, M-grouped contiguous and M-grouped masked references:
  decode exactly, scale per K block, accumulate in float64, round once.
* ``exact`` -- the same GEMM in exact rational arithmetic, for tiny shapes.
* ``ue8m0`` -- packing of exponent-only scales, four per int32 word.

Every function is pinned by CPU tests against closed forms, library decoders,
brute force, exact-rational golden cases and invariants; no function is
"parity unpinned".  tests/test_oracle_mutations.py plants one plausible mistake
at a time in these functions (reciprocal instead of division in the scale or
the quotient, a skipped fp32 rounding, ties away from zero, UE8M0 rounded down,
no amax floor, bf16 truncation or double rounding, K-block scale order, the B
scale index, a spurious factor, a dropped K block) and checks that a pin fails.
"""
from . import bf16, e4m3, exact, gemm, quant, ue8m0  # noqa: F401
