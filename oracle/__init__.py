"""fp64 CPU oracle for scaled-dot-product attention -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library and never
imports it; the product path never calls it.
"""
from .attention import sdpa_reference, allclose_report  # noqa: F401
from .backward import sdpa_backward_reference  # noqa: F401
