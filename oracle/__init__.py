"""CPU oracles of the action-expert denoise loop and of the VLM prefix prefill
(test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import it.
"""
from . import pi_ae_oracle  # noqa: F401
from . import prefill_oracle  # noqa: F401
