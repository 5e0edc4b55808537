"""MI355X (gfx950) cached flow-matching DiT step.

- ``diffusion_transformer_amd._lib``: ctypes binding of ``libdit.so`` (the C ABI in
  ``include/dit.h``); importing it fails loudly if the library is not built.
- ``diffusion_transformer_amd.runtime``: torch-held device memory and the sampler loop.
- ``diffusion_transformer_amd.synth``: seeded synthetic workloads.
- ``diffusion_transformer_amd.build``: builds ``libdit.so`` with hipcc for gfx950.
"""
__version__ = "0.1.0"
