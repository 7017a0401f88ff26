"""MI355X-native speculative-verify attention over a paged E4M3 KV cache.

The compute path is the HIP library ``libattn.so`` built from ``csrc/`` (see
``include/attn.h`` for its C ABI); ``attention`` is the thin ctypes binding
over it. Importing this package loads nothing; the library is loaded on first
use and a missing library raises instead of falling back to anything else.
"""
__all__ = ["attention", "workloads"]
