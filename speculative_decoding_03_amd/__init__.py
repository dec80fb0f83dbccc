"""MI355X-native greedy speculative decoding with an MTP drafter.

The HIP kernels and the C ABI live in ``csrc/`` (built into ``libspecdec.so``, declared in
``include/specdec.h``); ``engine`` is the thin Python binding over them.
"""

from . import _ffi as ffi  # noqa: F401
from ._ffi import (ACCEPT_COMMIT, BF16, F32, HEAD_CLUSTERED, HEAD_FULL, SpecdecError,  # noqa: F401
                   load)


def __getattr__(name):
    # the torch-based binding is imported lazily so that the ctypes layer loads without torch
    if name in ("Engine", "DeviceModel", "Shape", "pack_matrix", "KPolicy"):
        from . import engine
        return getattr(engine, name)
    raise AttributeError(name)
