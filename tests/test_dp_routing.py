"""Data-parallel routing over several radix trees (host only).

The native router (radix_route, driven by prefix_shared_kv_radix_amd/dp_sim.py)
against the oracle (oracle/routing.py): same worker for every request, same
admissions, slot rows and free lists per worker, bit for bit. The oracle's routing
is pinned by what its definition fixes: round robin is i mod n; least load keeps
every phase's shares within one request of each other; cache-aware routing, when
the balance rule does not fire, picks a worker holding the longest common prefix
with a sequence finished on it (brute force over the finished sequences, pools
large enough that nothing is evicted), and on branching workloads it keeps every
request with the worker holding its shared prefix, so the workers together reuse
exactly what one worker would (SGLang feature article §一 data-parallel attention,
§五 cache-aware load balancer, heading only).
"""
import random

import numpy as np
import pytest

from oracle.episode import run_episode
from oracle.routing import run_dp_episode
from prefix_shared_kv_radix_amd.dp_sim import run_dp
from workloads import Phase, Workload, _req, agent_branch, chat_tree, few_shot, tiny_shape

POLICIES = ["round_robin", "least_load", "cache_aware"]


def _fuzz(seed, n=40):
    rng = random.Random(seed)
    reqs = []
    for i in range(n):
        L = rng.randint(1, 12)
        toks = np.array([rng.randint(0, 2) for _ in range(L)], np.int32)
        outs = np.array([rng.randint(0, 2) for _ in range(2)], np.int32)
        reqs.append(_req(i, toks, np.arange(L) + 100 * i, outs, np.arange(2) + 100 * i + 50))
    phases, i = [], 0
    while i < n:
        k = rng.randint(1, 9)
        phases.append(Phase(list(range(i, min(n, i + k))), rng.choice(["fcfs", "lpf"]),
                            rng.randint(1, 4), rng.randint(0, 2), "host"))
        i += k
    return Workload("dp_fuzz", seed, tiny_shape(), rng.randint(24, 60), reqs, phases, 1, 1, 1)


def _compare(w, workers, policy, **kw):
    got = run_dp(w, workers, policy, **kw)
    ref = run_dp_episode(w, workers, policy, **kw)
    assert got.assignment == ref.assignment
    for g, r in zip(got.logs, ref.logs):
        assert len(g.rounds) == len(r.rounds)
        for gr, rr in zip(g.rounds, r.rounds):
            assert [a.rid for a in gr.admissions] == [a.rid for a in rr.admissions]
            for a, b in zip(gr.admissions, rr.admissions):
                assert a.prefix_len == b.prefix_len
                np.testing.assert_array_equal(a.row, b.row)
            np.testing.assert_array_equal(gr.decode_slots, rr.decode_slots)
        np.testing.assert_array_equal(g.free_list, r.free_list)
    return got, ref


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("workers", [2, 3, 8])
def test_native_matches_oracle_on_workloads(policy, workers):
    for w in (few_shot(2, tiny_shape(), 70, 30, 9, 3),
              agent_branch(4, tiny_shape(), 5, 60, 4, 20, 3, 4),
              chat_tree(13, tiny_shape(), 12, 5, 5, 30, 0.6)):
        _compare(w, workers, policy)


@pytest.mark.parametrize("seed", range(12))
def test_native_matches_oracle_on_fuzz_with_eviction(seed):
    w = _fuzz(seed)
    for policy in POLICIES:
        try:
            run_dp_episode(w, 3, policy, balance_abs=2, balance_rel=1.2, pool_factor=1.0)
        except RuntimeError:
            continue   # a pool too small for some round in this trace
        _compare(w, 3, policy, balance_abs=2, balance_rel=1.2, pool_factor=1.0)


def test_round_robin_and_least_load_shares():
    w = few_shot(2, tiny_shape(), 70, 29, 9, 0)
    rr = run_dp_episode(w, 4, "round_robin")
    order = [rid for ph in w.phases for rid in ph.rids]
    assert [rr.assignment[rid][0] for rid in order] == [i % 4 for i in range(len(order))]
    ll = run_dp_episode(w, 4, "least_load")
    for ph in w.phases:
        counts = np.bincount([ll.assignment[r][0] for r in ph.rids], minlength=4)
        assert counts.max() - counts.min() <= 1


def _lcp(a, b):
    n = 0
    while n < min(len(a), len(b)) and a[n] == b[n]:
        n += 1
    return n


@pytest.mark.parametrize("seed", range(8))
def test_cache_aware_picks_a_longest_prefix_worker(seed):
    """One request per phase (no balance rule can fire: loads are all zero), big
    pools: the chosen worker's longest common prefix with the sequences finished on it
    is the best over all workers."""
    rng = random.Random(500 + seed)
    reqs = []
    for i in range(30):
        L = rng.randint(1, 14)
        toks = np.array([rng.randint(0, 2) for _ in range(L)], np.int32)
        reqs.append(_req(i, toks, np.arange(L) + 100 * i, np.array([1], np.int32),
                         np.array([100 * i + 60])))
    phases = [Phase([i], "fcfs", 1, 1, "host") for i in range(30)]
    w = Workload("dp_lcp", seed, tiny_shape(), 10000, reqs, phases, 1, 1, 1)
    ep = run_dp_episode(w, 3, "cache_aware")
    done = [[] for _ in range(3)]
    for i in range(30):
        k, m = ep.assignment[i]
        best = [max([_lcp(reqs[i].tokens, s) for s in done[j]] + [0]) for j in range(3)]
        assert m == best[k] == max(best)
        assert k == min(j for j in range(3) if best[j] == max(best))   # ties: lower index
        done[k].append(w.full_tokens(i))


def test_cache_aware_keeps_branching_reuse():
    """Agent branching over 4 workers: every branch lands with its root, every fork
    with its branch, so the workers together reuse what one worker does; round robin
    scatters them and recomputes."""
    w = agent_branch(4, tiny_shape(), 8, 60, 4, 20, 3, 2)
    one = run_episode(w).hits()[1]
    ca = run_dp_episode(w, 4, "cache_aware")
    reused = sum(a.prefix_len for lg in ca.logs for r in lg.rounds for a in r.admissions)
    assert reused == one
    rr = run_dp_episode(w, 4, "round_robin")
    assert sum(a.prefix_len for lg in rr.logs for r in lg.rounds for a in r.admissions) < one
