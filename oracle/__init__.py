"""CPU oracle for the N:M structured-sparse GEMM path — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never calls it and shares no code
with it. See oracle.c for the citations of what each routine computes.
"""
from .oracle import *  # noqa: F401,F403
