"""MI355X-native batched prefill of a Qwen3-style decoder stack feeding a
multi-codebook audio head, and the head's delayed-codebook step.

The work runs in libhr.so (hand-written HIP kernels for gfx950 behind the C ABI
of include/hr.h and include/hr_ops.h); ``codebook_decode_amd.hr`` is its thin
ctypes binding.  Build with ``python -m codebook_decode_amd.build``.
"""
from . import hr  # noqa: F401

__all__ = ["hr"]
