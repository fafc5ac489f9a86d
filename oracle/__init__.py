"""CPU oracle for the radix-shared KV attention path.

TEST INFRASTRUCTURE. This package is a plain, slow, obviously correct
restatement of what the path computes, written from the pages' description:
  * ``radix``     slot pool, radix tree (match / split / insert / pin),
                  leaf-first LRU eviction, FCFS and longest-prefix-first order;
  * ``episode``   the request lifecycle over a workload script;
  * ``attention`` exact causal softmax attention per request in fp64;
  * ``blockhash`` the same request scripts through a 16-token block-hash-chain
                  prefix cache, for the token-level vs block-level reuse
                  comparison (``blockhash_report`` writes the stored table).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code with the HIP path and imports
nothing from it; the two meet only at the seeded inputs of ``workloads``.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
facts the pages and mathematics fix (see each test's docstring).
"""
from . import attention, blockhash, episode, radix  # noqa: F401
