"""MI355X-native paged attention (gfx950 HIP kernels behind a C ABI).

The native library ``libpa.so`` is loaded on first use; see ``api.py``.
"""
from .api import (  # noqa: F401
    PagedAttentionError,
    cache_write,
    check_copy_host,
    copy_blocks,
    decode,
    decode_shared,
    decode_shared_workspace_size,
    decode_workspace_size,
    library,
    set_kernel_timing_events,
    varlen_mixed,
    varlen_mixed_workspace_size,
    check_inputs_host,
)
from .engine import Engine  # noqa: F401,E402
