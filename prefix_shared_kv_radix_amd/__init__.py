"""MI355X-native attention over a radix-shared, token-granular KV slot pool.

Native library (libradix_attn.so, built by ``python -m prefix_shared_kv_radix_amd.build``):
  * host: slot pool, radix tree (token-level match, edge split, pinning,
    leaf-first LRU eviction), FCFS / longest-prefix-first ordering, and the
    shared-segment decode plan;
  * device (gfx950 HIP): KV store, extend attention (bf16 MFMA), decode
    attention (shared-segment MFMA + split-KV tail + LSE combine), MLA decode.
``_lib`` is the ctypes binding; ``runner`` sequences a workload through it.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
