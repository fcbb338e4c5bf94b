"""EntropyCache denoising step for MI355X (gfx950): C-ABI library + thin binding.

The compute path is libec.so (hand-written HIP for gfx950); this package only
marshals torch tensors into its C entry points (see lib.py) and holds a small
host-side runner (runner.py) that owns the device buffers of one sequence.
"""
from . import lib  # noqa: F401
