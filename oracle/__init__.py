"""FP64 CPU oracle for batched speculative-verify attention over a paged E4M3 KV cache.

This package is test infrastructure. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it. The
product path (the HIP library and its Python binding) never calls it, and the
oracle imports nothing from the product package.

What it computes follows these pages:

* "DFlash2 concurrent long-context attention, 2026-09-27" (design note), section
  "Why the single-request optimization was missing from concurrent decode":
  the kernel contract is E4M3 KV, FP16 queries, D = 256, six query heads per KV
  head, q8 verify batches, zero-length rows and padded requests stay safe.
* "SM70 attention and quantized projection coverage across TP sizes", section
  "Scope": on the GPU side the operands are FP16 and both products (scores and
  the weighted sum of values) accumulate in FP32; the oracle itself works in FP64.
* "perf(fa2): port decode GQA group-swap into d128 varlen launcher" (PR #48),
  PR description: the query heads of one KV group are packed together and read
  KV once per group (head h belongs to KV head h // G).

Parity status of each function is stated in its module header.
"""
from .e4m3 import decode_byte, decode_table
from .e5m2 import decode_byte as decode_e5m2_byte, decode_table as decode_e5m2_table
from .attention import verify_attention, partial_states, merge_partials

__all__ = ["decode_byte", "decode_table", "decode_e5m2_byte", "decode_e5m2_table", "verify_attention",
           "partial_states", "merge_partials"]
