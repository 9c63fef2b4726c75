"""Persistent batch-1 decode megakernel for AMD MI355X (gfx950).

The compute path is the C-ABI library libmk.so (include/mk.h) built from the
HIP sources in csrc/; `mk` is its ctypes binding.  PyTorch supplies device
memory and streams only.
"""
from .build import build as build_library  # noqa: F401
from .mk import (KVCache, MegaKernel, MkError, load_library, model_desc, upload_weights)  # noqa: F401
