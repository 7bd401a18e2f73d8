"""MI355X-native Gated DeltaNet-2 chunked prefill forward.

``chunk_fwd`` (in :mod:`.gdn2`) calls the C-ABI library ``libgdn2.so`` built
from ``csrc/`` for gfx950. Importing this package does not load the library;
the first call does, and raises if it is missing.
"""

__all__ = ["chunk_fwd", "last_error"]


def __getattr__(name):
    if name in __all__:
        from . import gdn2
        return getattr(gdn2, name)
    raise AttributeError(name)
