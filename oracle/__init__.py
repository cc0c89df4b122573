"""CPU oracle for tree speculative-sampling verification.

TEST INFRASTRUCTURE. Only tests/, the package smoke check and the benchmark's
CPU-baseline leg may import this package. It is independent of the HIP path
(include/specverify.h and the library behind it): the two share no code.
"""
from .verify import *  # noqa: F401,F403
