"""MI355X (gfx950) basis-synchronized online low-rank KV-cache compression.

The compute path lives in libiskv.so (HIP kernels + C ABI, include/iskv.h);
``binding`` is a thin ctypes layer over it.
"""
from .binding import (  # noqa: F401
    BF16, F32, Config, IskvCache, IskvError, Status, load_library, make_config, pack_state,
    state_bytes, strerror, unpack_state, workspace_bytes,
)
