"""MI355X-native action-expert flow-matching denoise loop.

The compute path is the HIP library ``libpi_ae.so`` built from ``csrc/``; the
Python binding in :mod:`flow_matching_action_amd.pi_ae` only marshals
arguments into its C-ABI.  :mod:`flow_matching_action_amd.inputs` generates the
seeded synthetic workloads.
"""
__all__ = ["inputs", "pi_ae"]
