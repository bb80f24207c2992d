"""CPU oracle for block-scaled low-bit fused attention (float64, numpy).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU path never does, and the
oracle imports nothing from the GPU path. Every function follows a passage of
the reference pages (cited in each module) and the readings listed in the
design notes; the tests pin it against closed forms, library routines,
invariants and a pure-Python brute force.

Parity status: every function here has at least one independent pin (see
tests/test_*_oracle.py); no function is parity-unpinned.
"""
from . import attention, decode, formats, outlier, quant, selection  # noqa: F401
