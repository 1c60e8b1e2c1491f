"""MI355X-native forward of a MOSS-Image-style DiT denoiser block.

The compute path is the HIP library ``libmoss.so`` (built from ``csrc/``)
behind the C ABI declared in ``include/moss.h``; ``moss`` is its thin ctypes
binding.  ``synth`` makes the seeded synthetic inputs.
"""
__all__ = ["synth", "moss"]
