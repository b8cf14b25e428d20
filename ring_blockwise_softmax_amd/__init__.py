"""Exact blockwise ring attention for MI355X (gfx950).

The computation runs in ``libra.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/ra.h``); this package is its thin binding.  Torch
supplies device memory and streams only.

Entry points (same names as the C ABI, without the ``ra_`` prefix):
``block_attn_fwd``, ``merge``, ``ring_forward``, ``ring_plan`` and the
workspace / profiling helpers.  Importing the package does not load the
library; the first call does, and fails loudly if it is missing.
"""

from .api import (  # noqa: F401
    block_attn_fwd,
    block_attn_fwd_noalloc,
    block_attn_workspace_bytes,
    merge,
    ring_forward,
    ring_workspace_bytes,
    ring_plan,
    RingRunner,
    profile_enable,
    profile_read,
)
from ._lib import RaError  # noqa: F401
