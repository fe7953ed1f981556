"""Dynamic block-sparse self-attention for video DiTs on MI355X (gfx950).

The hot path runs in ``libsparse_attn.so`` (hand-written HIP kernels behind
the C-ABI in ``include/sparse_attn.h``); :mod:`.binding` marshals torch
tensors into it.  :mod:`.synth` draws the seeded synthetic inputs.
"""
from . import binding  # noqa: F401  (loads the library lazily, on first call)

__all__ = ["binding"]
