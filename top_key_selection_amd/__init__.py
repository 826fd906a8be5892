"""MI355X (gfx950) sparse-attention indexer + top-k: flat DSA-style scan and
HISA hierarchical block filter, behind the C ABI of include/tks.h.

The binding (``top_key_selection_amd.tks``) loads ``libtks.so`` on first
use; build it with ``python -m top_key_selection_amd.build``.
"""
from . import tks  # noqa: F401
from .tks import (FORCE_FIRST, FORCE_LOCAL, KEY_BF16, KEY_FP8_E4M3FN, Shape,  # noqa: F401
                  TksError)
