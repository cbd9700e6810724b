"""CPU oracle for the NVFP4 quantized-linear hot path (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
this package.  The product library never imports or links it, and it shares
no code with the HIP sources.
"""
from .oracle import *  # noqa: F401,F403
