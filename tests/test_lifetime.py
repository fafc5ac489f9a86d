"""Lifetime of the native pool and tree objects (CPU only).

A tree returns its cached slots to its pool when it is destroyed, so the pool's
memory must still exist then, whichever of the two the caller destroys first (a
garbage collector breaking a reference cycle picks the order itself). Each case
runs in a child process so that a use-after-free shows up as a crash (a large
pool's free list is unmapped when freed) instead of taking the test runner down.
"""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PRELUDE = textwrap.dedent("""
    import gc, sys
    import numpy as np
    sys.path.insert(0, %r)
    from prefix_shared_kv_radix_amd import _lib
    N = 1 << 22          # a 4M-slot pool: its free list is unmapped when freed
""" % ROOT)


def _run(body):
    r = subprocess.run([sys.executable, "-c", PRELUDE + textwrap.dedent(body)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, f"child exited with {r.returncode}:\n{r.stdout}"
    return r.stdout


def test_pool_destroyed_before_tree_c_abi():
    """radix_kv_pool_destroy, then radix_tree_destroy on a tree that still caches slots."""
    out = _run("""
        lib = _lib.load()
        pool = _lib.KVPool(N)
        tree = _lib.RadixTree(pool)
        slots = tree.alloc(1000)
        tree.insert(np.arange(1000, dtype=np.int32), slots)
        ph, th = pool.h, tree.h
        pool.h = tree.h = None                # the wrappers no longer own the handles
        lib.radix_kv_pool_destroy(ph)
        lib.radix_tree_destroy(th)            # releases 1000 slots into the pool
        print("ok")
    """)
    assert out.strip().endswith("ok")


def test_tree_keeps_working_after_pool_handle_released():
    """The tree's own hold on the pool keeps allocation and eviction valid."""
    out = _run("""
        lib = _lib.load()
        pool = _lib.KVPool(3000)
        tree = _lib.RadixTree(pool)
        s = tree.alloc(2000)
        tree.insert(np.arange(2000, dtype=np.int32), s)
        ph = pool.h
        pool.h = None
        lib.radix_kv_pool_destroy(ph)
        more = tree.alloc(2500)               # evicts the cached 2000 tokens
        assert len(set(more.tolist())) == 2500
        assert tree.stats().evicted_tokens_total == 2000
        tree.close()
        print("ok")
    """)
    assert out.strip().endswith("ok")


def test_pool_and_tree_in_a_reference_cycle():
    """Pool and tree die together in a cycle, collected by gc in its own order."""
    out = _run("""
        for rep in range(4):
            pool = _lib.KVPool(N)
            tree = _lib.RadixTree(pool)
            slots = tree.alloc(1000)
            tree.insert(np.arange(1000, dtype=np.int32) + rep, slots)
            holder = {"pool": pool, "tree": tree}
            pool.cycle = holder
            tree.cycle = holder
            del pool, tree, holder, slots
            gc.collect()
        print("ok")
    """)
    assert out.strip().endswith("ok")
