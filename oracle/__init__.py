"""CPU oracle for the weight-only quantized GEMM and its MoE variant.

Test infrastructure only: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The library under test
never imports this package, and this package never imports the library.
"""
from .qref import *  # noqa: F401,F403
