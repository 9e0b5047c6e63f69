"""CPU oracle of the TTT-E2E prefill: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may use it.
"""
from .ttt_oracle import Oracle, prefill  # noqa: F401
