"""Pins of the oracle's tree, pool, eviction and scheduler against what the pages fix.

Sources: page "49 · RadixAttention, eviction và cache churn" (§2 two-request
split and multi-turn reuse, §4 eviction rules, §5 ordering and its theorem,
§6 churn numbers) and the SGLang overview (nine-step example).
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle.episode import run_episode
from oracle.radix import PoolError, RadixTree, SlotPool, schedule_order
from workloads import Phase, Workload, _req, cyclic_stream, tiny_shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _admit(tree, toks):
    m, cached, node = tree.match(toks)
    tree.lock(node)
    new = tree.alloc(len(toks) - m)
    assert new is not None
    return m, np.concatenate([cached, np.asarray(new, np.int32)]).astype(np.int32), node


def _finish(tree, toks, row, m, node):
    c = tree.insert(toks, row)
    if c > m:
        tree.pool.release(row[m:c])
    tree.unlock(node)
    return c


# ---------------------------------------------------------------- page 4 §2
def test_two_request_split():
    g = _load("two_request_split_page4.json")
    S, Q1, Q2 = g["system_prompt"], g["q1"], g["q2"]
    pool = SlotPool(g["pool_slots"])
    tree = RadixTree(pool)
    r1 = S + Q1
    m1, row1, n1 = _admit(tree, r1)
    assert m1 == 0
    _finish(tree, r1, row1, m1, n1)
    # R1 is a single path from the root
    assert len(tree.root.children) == 1
    only = next(iter(tree.root.children.values()))
    assert list(only.key) == r1 and not only.children
    r2 = S + Q2
    free_before = pool.num_free()
    m2, row2, n2 = _admit(tree, r2)
    assert m2 == g["expected_r2"]["matched"]
    assert free_before - pool.num_free() == g["expected_r2"]["new_slots"]   # only Q2 computed
    assert list(row2[:len(S)]) == list(row1[:len(S)])                     # stem slots reused
    _finish(tree, r2, row2, m2, n2)
    assert len(tree.root.children) == g["expected_tree"]["root_children"]
    stem = next(iter(tree.root.children.values()))
    assert len(stem.key) == g["expected_tree"]["stem_len"]
    assert sorted(len(c.key) for c in stem.children.values()) == g["expected_tree"]["branch_lens"]
    assert list(stem.value) == list(row1[:len(S)])


def test_finished_request_with_outputs_stays():
    """Turn t+1 finds all of turn t, including what turn t generated (page 4 §2)."""
    pool = SlotPool(100)
    tree = RadixTree(pool)
    prompt = [5, 6, 7, 8]
    m, row, node = _admit(tree, prompt)
    outs = [40, 41, 42]
    dec = tree.alloc(len(outs))
    full_row = np.concatenate([row, dec]).astype(np.int32)
    _finish(tree, prompt + outs, full_row, m, node)
    nxt = prompt + outs + [77, 78]
    m2, row2, _ = _admit(tree, nxt)
    assert m2 == len(prompt) + len(outs)
    assert list(row2[:m2]) == list(full_row)


def test_match_equals_brute_force_longest_prefix():
    """m equals the longest common prefix with any resident root-to-node path."""
    rng = random.Random(7)
    pool = SlotPool(10_000)
    tree = RadixTree(pool)
    seqs = []
    for _ in range(60):
        if seqs and rng.random() < 0.7:
            base = rng.choice(seqs)
            cut = rng.randint(0, len(base))
            s = base[:cut] + [rng.randint(0, 3) for _ in range(rng.randint(0, 6))]
        else:
            s = [rng.randint(0, 3) for _ in range(rng.randint(1, 8))]
        expect = max([0] + [_lcp_list(s, t) for t in seqs])
        assert tree.peek(s) == expect
        m, row, node = _admit(tree, s)
        assert m == expect
        _finish(tree, s, row, m, node)
        seqs.append(s)


def _lcp_list(a, b):
    k = 0
    while k < len(a) and k < len(b) and a[k] == b[k]:
        k += 1
    return k


# ---------------------------------------------------------------- page 4 §6
def _hits(log):
    return log.hits()[0]


def test_churn_cyclic_zero_of_ten():
    g = _load("churn_page4.json")
    w = cyclic_stream(4, tiny_shape(), g["distinct_prefixes"], 2048, 2, g["cache_prefixes"],
                      "cyclic", "fcfs")
    log = run_episode(w)
    assert sum(len(r.admissions) for r in log.rounds) == g["requests"]
    assert _hits(log) == g["cyclic_hits"]


def test_churn_grouped_five_of_ten():
    g = _load("churn_page4.json")
    w = cyclic_stream(4, tiny_shape(), g["distinct_prefixes"], 2048, 2, g["cache_prefixes"],
                      "grouped", "fcfs")
    assert _hits(run_episode(w)) == g["grouped_hits"]


def test_churn_lpf_with_all_queued_recovers_grouping():
    """Longest-prefix-first over the queued cyclic stream serves it grouped (5/10)."""
    g = _load("churn_page4.json")
    w = cyclic_stream(4, tiny_shape(), g["distinct_prefixes"], 2048, 2, g["cache_prefixes"],
                      "cyclic", "lpf")
    assert _hits(run_episode(w)) == g["grouped_hits"]


def test_churn_sweep_200_cycles():
    """0 % until the cache holds the whole working set, then all but the cold misses."""
    g = _load("churn_page4.json")
    for k in range(1, 7):
        w = cyclic_stream(4, tiny_shape(), 5, 8, 200, k, "cyclic", "fcfs")
        hits = _hits(run_episode(w))
        if k < 5:
            assert hits / 1000 == g["sweep_below_working_set_hit_rate"], (k, hits)
        else:
            assert hits == 995 and hits / 1000 >= g["sweep_at_working_set_hit_rate_min"], (k, hits)


# ---------------------------------------------------------------- page 4 §5
def _workload_from_prompts(prompts, pool_slots, policy, batch_limit=1):
    reqs = [_req(i, np.asarray(p, np.int32), np.arange(len(p), dtype=np.int64) + 1000 * i)
            for i, p in enumerate(prompts)]
    return Workload("t", 0, tiny_shape(), pool_slots, reqs,
                    [Phase(list(range(len(prompts))), policy, batch_limit, 0, "host")],
                    1, 1, 1)


def _computed_tokens(log):
    return sum(a.prompt_len - a.prefix_len for r in log.rounds for a in r.admissions)


def test_nine_requests_one_prefix_cache():
    """Cache of one prefix, 3 prefixes x 3 requests interleaved: FCFS 0/9, LPF 6/9."""
    X, Y, Z = [1] * 6, [2] * 6, [3] * 6
    prompts = [X, Y, Z] * 3
    fc = run_episode(_workload_from_prompts(prompts, 6, "fcfs"))
    lp = run_episode(_workload_from_prompts(prompts, 6, "lpf"))
    assert _hits(fc) == 0
    assert _hits(lp) == 6


def test_lpf_optimal_brute_force():
    """For a fixed batch and a cache holding the longest request, LPF computes the
    fewest tokens: equal to the distinct-prefix (union trie) count and to the minimum
    over every arrival order served first-come-first-served."""
    rng = random.Random(11)
    for trial in range(150):
        n = rng.randint(2, 6)
        prompts = [[rng.randint(0, 2) for _ in range(rng.randint(1, 5))] for _ in range(n)]
        cap = max(len(p) for p in prompts) + rng.randint(0, 3)
        union = len({tuple(p[:i]) for p in prompts for i in range(1, len(p) + 1)})
        lpf = _computed_tokens(run_episode(_workload_from_prompts(prompts, cap, "lpf")))
        best = min(_computed_tokens(run_episode(_workload_from_prompts([prompts[i] for i in perm],
                                                                       cap, "fcfs")))
                   for perm in itertools.permutations(range(n)))
        assert lpf == best == union, (prompts, cap)


def test_schedule_order_is_stable_on_ties():
    pool = SlotPool(50)
    tree = RadixTree(pool)
    m, row, node = _admit(tree, [1, 2, 3])
    _finish(tree, [1, 2, 3], row, m, node)
    prompts = [[9], [1, 2], [8], [1, 2, 3, 4], [1, 2, 5]]
    assert schedule_order(tree, prompts, "fcfs") == [0, 1, 2, 3, 4]
    assert schedule_order(tree, prompts, "lpf") == [3, 1, 4, 0, 2]


# ---------------------------------------------------------------- page 4 §4
def test_eviction_rules_on_random_traces():
    """Pinned nodes never go; only leaves go; among unpinned leaves the least recently
    used goes first; a parent becomes a candidate once childless; slots are conserved."""
    for seed in range(25):
        rng = random.Random(seed)
        pool = SlotPool(rng.randint(12, 40))
        tree = RadixTree(pool)
        orig_release = pool.release

        def checked_release(slots, _tree=tree, _orig=orig_release):
            slots = [int(s) for s in slots]
            owner = [n for n in _tree.nodes() if list(n.value) == slots]
            if owner:     # a node being evicted
                n = owner[0]
                assert not n.children and n.lock == 0
                leaves = [x for x in _tree.nodes() if not x.children and x.lock == 0]
                assert n.tick == min(x.tick for x in leaves)
            _orig(slots)
        pool.release = checked_release
        running = []
        for step in range(120):
            if running and (rng.random() < 0.45 or len(running) > 3):
                toks, row, m, node = running.pop(rng.randrange(len(running)))
                _finish(tree, toks, row, m, node)
            else:
                toks = [rng.randint(0, 2) for _ in range(rng.randint(1, 7))]
                m, cached, node = tree.match(toks)
                tree.lock(node)
                new = tree.alloc(len(toks) - m)
                if new is None:
                    tree.unlock(node)
                else:
                    running.append((toks, np.concatenate([cached, np.asarray(new, np.int32)]), m, node))
            # conservation: free + cached + running-owned new slots = all, disjoint
            owned = [s for (t, row, m, nd) in running for s in row[m:]]
            cached_slots = [int(s) for n in tree.nodes() for s in n.value]
            allslots = list(pool.free) + cached_slots + [int(s) for s in owned]
            assert sorted(allslots) == list(range(pool.num_slots))
            # pinned paths are intact
            for (t, row, m, nd) in running:
                assert tree.peek(t) >= m


def test_alloc_is_all_or_nothing():
    pool = SlotPool(10)
    tree = RadixTree(pool)
    m, row, node = _admit(tree, [1, 2, 3, 4, 5, 6])
    before = (list(pool.free), tree.tick)
    assert tree.alloc(5) is None        # 4 free, 0 evictable (pinned)
    assert (list(pool.free), tree.tick) == before
    _finish(tree, [1, 2, 3, 4, 5, 6], row, m, node)
    got = tree.alloc(10)                # now evictable
    assert got is not None and len(got) == 10


def test_pool_fifo_and_bad_frees():
    pool = SlotPool(6)
    assert pool.alloc(3) == [0, 1, 2]
    pool.release([1, 0])
    assert list(pool.free) == [3, 4, 5, 1, 0]
    with pytest.raises(PoolError):
        pool.release([3])      # already free
    with pytest.raises(PoolError):
        pool.release([6])      # out of range
    with pytest.raises(PoolError):
        pool.release([2, 2])   # double in one call
    assert pool.alloc(6) is None


# ---------------------------------------------------- SGLang overview, 9 steps
def test_nine_step_evolution():
    """Constructed token script (pool of 19 slots) reproducing the events of the
    nine-step example: a chat turn as one edge; the next turn hung below it; a second
    session splitting the first at the shared system prompt; an LRU eviction of the
    first session's newest node making room for the second session's next turn,
    which hangs below the second session's node; a few-shot request with no shared
    prefix as a new branch of the root; a few-shot batch splitting that node; a new
    message of session 1 evicting all of session 2; sampling more answers evicting
    several nodes. The figure's token strings are not in the text, so the tokens and
    capacity are constructed; the events are the page's."""
    sysp = [1, 1, 1, 1]
    u1 = [2, 2, 2, 2]
    pool = SlotPool(19)
    tree = RadixTree(pool)

    def serve(prompt, outs):
        m, row, node = _admit(tree, prompt)
        dec = tree.alloc(len(outs))
        assert dec is not None
        _finish(tree, prompt + outs, np.concatenate([row, dec]).astype(np.int32), m, node)
        return m

    # step 1: empty
    assert not tree.root.children
    # step 2: system prompt + user message + answer become one edge
    s1 = sysp + u1
    serve(s1, [3, 3])
    assert len(tree.root.children) == 1
    e = next(iter(tree.root.children.values()))
    assert list(e.key) == s1 + [3, 3] and not e.children
    # step 3: the next turn reuses the first and hangs a new node below it
    m = serve(s1 + [3, 3, 4, 4], [5, 5])
    assert m == len(s1) + 2 and len(e.children) == 1
    # step 4: a second session splits that edge at the system prompt
    serve(sysp + [6, 6], [7, 7])
    stem = next(iter(tree.root.children.values()))
    assert list(stem.key) == sysp and len(stem.children) == 2
    assert len(tree.evict_log) == 0
    # step 5: session 2 continues; the pool is short, one node of session 1 goes (its
    # least recently used leaf) and the new turn hangs below session 2's node
    s2_next = sysp + [6, 6, 7, 7, 8]
    serve(s2_next, [9, 9])
    assert len(tree.evict_log) == 1
    assert tree.peek(s1 + [3, 3, 4, 4, 5, 5]) == len(s1) + 2     # session 1's turn 2 gone
    assert tree.peek(s2_next + [9, 9]) == len(s2_next) + 2
    s2_node = stem.children[6]
    assert list(s2_node.key) == [6, 6, 7, 7] and len(s2_node.children) == 1
    # step 6: a few-shot request with no shared prefix becomes a new branch of the root
    shots = [20, 21, 22]
    serve(shots + [30], [31])
    assert len(tree.root.children) == 2
    assert tree.peek(s2_next + [9, 9]) == len(s2_next) + 2        # session 2 untouched
    # step 7: a batch of few-shot questions sharing the examples splits that node
    n_ev = len(tree.evict_log)
    running = []
    for q in (40, 41, 42):
        m, row, node = _admit(tree, shots + [q])
        running.append((shots + [q], row, m, node))
    for t, row, m, node in running:
        _finish(tree, t, row, m, node)
    fs = tree.root.children[20]
    assert list(fs.key) == shots and len(fs.children) == 4
    assert len(tree.evict_log) == n_ev
    # step 8: a new message from session 1 evicts every node of session 2
    n_ev = len(tree.evict_log)
    serve(s1 + [3, 3, 10], [11])
    assert tree.peek(s2_next) == len(sysp)
    assert len(tree.evict_log) - n_ev >= 2
    assert tree.peek(shots + [40]) == len(shots) + 1
    # step 9: sampling more answers for a question evicts several nodes
    n_ev = len(tree.evict_log)
    running = []
    for k in range(2):
        m, row, node = _admit(tree, shots + [40])
        dec = tree.alloc(2)
        assert dec is not None
        running.append((shots + [40] + [50 + k] * 2, np.concatenate([row, dec]).astype(np.int32), m, node))
    for t, row, m, node in running:
        _finish(tree, t, row, m, node)
    assert len(tree.evict_log) - n_ev >= 2
