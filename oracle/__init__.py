"""CPU oracle for the DSA prefill hot path -- TEST INFRASTRUCTURE, not part of the product.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
It shares no code with the HIP library and never imports it.
"""
from .dsa_oracle import *  # noqa: F401,F403
