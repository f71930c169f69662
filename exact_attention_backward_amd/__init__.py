"""Exact attention backward for AMD MI355X (gfx950).

The computation lives in the HIP library ``libattnbwd.so`` (C ABI in
``include/attn_bwd.h``); ``api`` binds it for torch tensors.  Build the library
with ``python -m exact_attention_backward_amd.build``.
"""

from . import _lib  # noqa: F401
from . import api  # noqa: F401

__all__ = ["api"]
