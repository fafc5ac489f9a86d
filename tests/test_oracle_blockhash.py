"""The block-hash prefix cache replay (oracle/blockhash.py) against what fixes it.

Page "49 · RadixAttention, eviction và cache churn", §3: vLLM's prefix caching
matches a chain of block hashes at 16-token granularity, RadixAttention matches
token by token; both share by reference count and evict least recently used
first. Pins:
  * brute force on tiny traces without eviction: a request reuses
    16 * floor(max_j min(LCP(prompt, seq_j), cached_j) / 16) tokens, where seq_j
    runs over the sequences finished before it and cached_j is the full-block part
    of seq_j; the radix tree reuses max_j LCP(prompt, seq_j) on the same trace;
  * block-aligned sharing (every shared prefix a multiple of 16 tokens) reuses
    exactly what the tree reuses;
  * the churn example of §6 (5 prefixes cycling through a cache of 4: 0/10;
    grouped: 5/10) holds for the block cache too, since both evict LRU;
  * block conservation at the end of every episode;
  * the stored comparison on the workload traces (tests/golden/blockhash_vs_radix.json,
    written by oracle/blockhash_report.py) for the traces that replay in seconds.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle.blockhash import run_block_episode
from oracle.episode import run_episode
from workloads import Phase, Workload, _req, config, few_shot, tiny_shape

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "blockhash_vs_radix.json")


def lcp(a, b):
    n = 0
    while n < min(len(a), len(b)) and a[n] == b[n]:
        n += 1
    return n


def _single_request_trace(seed, alphabet=2, n=25, pool=100000):
    rng = random.Random(seed)
    reqs = []
    for i in range(n):
        L = rng.randint(1, 70)
        toks = np.array([rng.randint(0, alphabet - 1) for _ in range(L)], np.int32)
        nd = rng.randint(0, 20)
        outs = np.array([rng.randint(0, alphabet - 1) for _ in range(nd)], np.int32)
        reqs.append(_req(i, toks, np.arange(L) + 1000 * i, outs, np.arange(nd) + 1000 * i + 500))
    phases = [Phase([i], "fcfs", 1, len(reqs[i].out_tokens), "host") for i in range(n)]
    return Workload("blk_fuzz", seed, tiny_shape(), pool, reqs, phases, 1, 1, 1)


@pytest.mark.parametrize("seed", range(30))
def test_brute_force_reuse_without_eviction(seed):
    w = _single_request_trace(seed)
    blk = run_block_episode(w)
    rad = run_episode(w)
    done = []
    for a, r in zip(blk.admissions, (x for rnd in rad.rounds for x in rnd.admissions)):
        assert a.rid == r.rid
        p = w.requests[a.rid].tokens
        best_tok = max([lcp(p, s) for s in done] + [0])
        best_blk = max([min(lcp(p, s), 16 * (len(s) // 16)) for s in done] + [0])
        assert r.prefix_len == best_tok
        assert a.reused == 16 * (best_blk // 16)
        done.append(w.full_tokens(a.rid))
    assert blk.evicted_blocks == 0
    assert blk.free_blocks + blk.cached_blocks == blk.num_blocks


def test_block_aligned_sharing_equals_radix():
    """Shared prefix 320 tokens, questions of 48: every request reuses the prefix in
    both caches, request by request."""
    w = few_shot(3, tiny_shape(), 320, 12, 48, 0)
    blk = run_block_episode(w)
    rad = run_episode(w)
    got = {a.rid: a.reused for a in blk.admissions}
    for rnd in rad.rounds:
        for a in rnd.admissions:
            assert got[a.rid] == a.prefix_len


def test_unaligned_prefix_loses_the_partial_block():
    """A 100-token shared prefix: the tree reuses 100 tokens, the block cache 96."""
    w = few_shot(3, tiny_shape(), 100, 6, 20, 0)
    blk = run_block_episode(w)
    assert [a.reused for a in blk.admissions] == [0] + [96] * 6


@pytest.mark.parametrize("variant,hits", [("cyclic", 0), ("grouped", 5), ("cyclic_lpf", 5)])
def test_churn_example_holds_for_blocks(variant, hits):
    assert run_block_episode(config(4, variant)).hits()[0] == hits


@pytest.mark.parametrize("seed", range(10))
def test_blocks_conserved_under_eviction(seed):
    """Tight pools force eviction; every pool block ends free or cached."""
    rng = random.Random(100 + seed)
    reqs = []
    for i in range(30):
        L = rng.randint(10, 90)
        toks = np.array([rng.randint(0, 1) for _ in range(L)], np.int32)
        reqs.append(_req(i, toks, np.arange(L) + 1000 * i, np.array([1, 0, 1], np.int32),
                         np.arange(3) + 1000 * i + 500))
    phases = [Phase(list(range(i, min(30, i + 3))), rng.choice(["fcfs", "lpf"]), 2, 3, "host")
              for i in range(0, 30, 3)]
    w = Workload("blk_tight", seed, tiny_shape(), 16 * 12, reqs, phases, 1, 1, 1)
    log = run_block_episode(w)
    assert log.evicted_blocks > 0
    assert len(log.admissions) == 30
    assert log.num_blocks == 12
    assert log.free_blocks + log.cached_blocks == log.num_blocks


def test_golden_comparison_on_workload_traces():
    with open(GOLDEN) as f:
        gold = {row["workload"]: row for row in json.load(f)["traces"]}
    for n, v in [(2, ""), (3, "A"), (4, "cyclic"), (4, "grouped"), (4, "cyclic_lpf")]:
        w = config(n, v)
        row = gold[w.name]
        assert run_episode(w).hits()[1] == row["radix"]["reused_tokens"], w.name
        assert run_block_episode(w).hits()[1] == row["block16"]["reused_tokens"], w.name
    # token-level matching never reuses less than block matching on these traces
    for row in gold.values():
        assert row["radix"]["reused_tokens"] >= row["block16"]["reused_tokens"]
