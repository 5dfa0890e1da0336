"""MI355X-native streamed NF4 + LoRA linear (gfx950).

The compute lives in liblnf4.so (HIP kernels behind a C ABI, include/lnf4.h);
``lnf4`` is its thin ctypes binding and ``stack`` drives a layer-streamed step
through it.
"""
from . import lnf4  # noqa: F401

__all__ = ["lnf4"]
