"""MI355X (gfx950) sparse embedding + DIN attention forward.

The computation lives in librec.so (HIP, built from csrc/ by
`python -m sparse_embedding_din_amd.build`); `rec` is its ctypes binding and
`pipeline` strings the four C-ABI calls into one forward over device buffers.
"""
from . import rec  # noqa: F401

__all__ = ["rec"]
