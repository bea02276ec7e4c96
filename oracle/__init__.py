"""CPU oracle of the action-expert denoise loop (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import it.
"""
from . import pi_ae_oracle  # noqa: F401
