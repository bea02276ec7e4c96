"""CPU oracles of the action-expert denoise loop, the VLM prefix prefill and the
vision encoder (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import it.
"""
from . import pi_ae_oracle  # noqa: F401
from . import prefill_oracle  # noqa: F401
from . import vision_oracle  # noqa: F401
