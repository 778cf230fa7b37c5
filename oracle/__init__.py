"""CPU oracle for one training step of a small bias-free decoder.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it.

Everything is plain numpy in float64; matrix products are library calls, every
other step is written out from its definition.  See ``oracle/model.py``.
"""
from .model import *  # noqa: F401,F403
from .model import __all__  # noqa: F401
from .kvcache import kv_cache_new, forward_cached  # noqa: F401

__all__ = list(__all__) + ["kv_cache_new", "forward_cached"]
