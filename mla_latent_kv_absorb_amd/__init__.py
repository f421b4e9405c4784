"""MI355X-native MLA absorb attention and latent-KV expansion.

The compute runs in hand-written HIP kernels for gfx950 behind a C-ABI library
(``libmla_absorb.so``, declared in ``include/mla_absorb.h``).  ``binding`` is a thin
ctypes layer over it; ``workloads`` draws seeded synthetic inputs.
"""
__all__ = ["binding", "workloads"]
