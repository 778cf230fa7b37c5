"""MI355X (gfx950) training step for a small bias-free decoder.

The compute path is libslt.so (HIP kernels behind a C ABI, include/slt.h);
``binding`` marshals arguments to it and ``trainer`` owns the device buffers
of one model (torch is used only to allocate memory and for the stream).
"""
from . import binding  # noqa: F401
from .binding import SltError, make_config  # noqa: F401
