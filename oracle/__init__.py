"""fp64 CPU oracle for paged attention, the KV-cache write and block copies (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library.
"""
from .oracle import build, cache_write, copy_blocks, paged_attention, read_counts, bf16_to_float64  # noqa: F401
