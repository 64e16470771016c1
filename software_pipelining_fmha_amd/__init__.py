"""MI355X-native fused multi-head attention forward pass.

The product is the C-ABI library `libfmha.so` (hand-written HIP for gfx950,
declared in include/fmha.h). `software_pipelining_fmha_amd.fmha` is its
Python binding. `software_pipelining_fmha_amd.inputs` draws the seeded
synthetic workloads.
"""
__all__ = ["fmha", "inputs"]
