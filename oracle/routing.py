"""Oracle: data-parallel routing over several workers, each with its own pool and tree.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The SGLang feature article spreads batches over independent data-parallel attention
workers so that KV is not stored twice (§一) and names a cache-aware load balancer
(§五, heading only). The pages give no rule, so the reading below is the library's:
  * round robin: worker i mod n for the i-th routed request;
  * least load: the worker with the fewest requests queued so far in the phase
    (lower index on ties);
  * cache-aware: when the queued loads are imbalanced (max - min > balance_abs and
    max > balance_rel * min) the least loaded worker; otherwise the worker whose tree
    holds the longest cached prefix of the prompt (peek, nothing changes), ties to
    the smaller load, then the lower index.
Each phase's requests are routed one by one against the trees as they stand at the
start of the phase; then every worker serves its share of the phase in rounds, the
same lifecycle as oracle.episode (order, admit, decode slots, insert, unpin).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

from .episode import Admission, EpisodeLog, Round
from .radix import RadixTree, SlotPool, schedule_order


def route(peeks, loads, policy: str, balance_abs: int, balance_rel: float, rr: int) -> int:
    n = len(loads)
    if policy == "round_robin":
        return rr % n
    least = min(range(n), key=lambda i: (loads[i], i))
    if policy == "least_load":
        return least
    if policy != "cache_aware":
        raise ValueError(policy)
    hi, lo = max(loads), min(loads)
    if hi - lo > balance_abs and float(hi) > balance_rel * float(lo):
        return least
    return min(range(n), key=lambda i: (-peeks[i], loads[i], i))


def _serve_phase(tree: RadixTree, reqs, p_idx, ph, rids, log: EpisodeLog) -> None:
    waiting = list(rids)
    while waiting:
        order = schedule_order(tree, [reqs[r].tokens for r in waiting], ph.policy)
        waiting = [waiting[i] for i in order]
        admitted, nodes = [], []
        for rid in waiting:
            if len(admitted) >= ph.batch_limit:
                break
            toks = reqs[rid].tokens
            m, cached, node = tree.match(toks)
            tree.lock(node)
            new = tree.alloc(len(toks) - m)
            if new is None:
                tree.unlock(node)
                break
            row = np.concatenate([cached, np.asarray(new, np.int32)]).astype(np.int32)
            admitted.append(Admission(rid, m, len(toks), row))
            nodes.append(node)
        if not admitted:
            raise RuntimeError(f"request {waiting[0]} cannot be admitted into an idle pool")
        taken = {a.rid for a in admitted}
        waiting = [r for r in waiting if r not in taken]
        dec = np.zeros((ph.n_decode, len(admitted)), np.int32)
        for s in range(ph.n_decode):
            for b in range(len(admitted)):
                got = tree.alloc(1)
                if got is None:
                    raise RuntimeError("pool exhausted during decode")
                dec[s, b] = got[0]
        counts = np.zeros(len(admitted), np.int64)
        for b, (a, node) in enumerate(zip(admitted, nodes)):
            r = reqs[a.rid]
            seq = np.concatenate([r.tokens, r.out_tokens[:ph.n_decode]])
            full_row = np.concatenate([a.row, dec[:, b]]).astype(np.int32)
            c = tree.insert(seq, full_row)
            tree.pool.release(full_row[a.prefix_len:c])
            tree.unlock(node)
            counts[b] = c
        log.rounds.append(Round(p_idx, admitted, dec, counts))


@dataclass
class DPEpisode:
    assignment: Dict[int, Tuple[int, int]] = field(default_factory=dict)  # rid -> (worker, peek)
    logs: List[EpisodeLog] = field(default_factory=list)
    trees: List[RadixTree] = field(default_factory=list)


def run_dp_episode(workload, workers: int, policy: str, balance_abs: int = 32,
                   balance_rel: float = 1.5, pool_factor: float = 2.0) -> DPEpisode:
    """Each worker's pool holds pool_factor x the workload's pool_slots."""
    trees = [RadixTree(SlotPool(int(workload.pool_slots * pool_factor))) for _ in range(workers)]
    out = DPEpisode(logs=[EpisodeLog() for _ in range(workers)], trees=trees)
    rr = 0
    reqs = workload.requests
    for p_idx, ph in enumerate(workload.phases):
        loads = [0] * workers
        share: List[List[int]] = [[] for _ in range(workers)]
        for rid in ph.rids:
            peeks = [t.peek(reqs[rid].tokens) for t in trees]
            k = route(peeks, loads, policy, balance_abs, balance_rel, rr)
            rr += 1
            share[k].append(rid)
            loads[k] += 1
            out.assignment[rid] = (k, peeks[k])
        for k in range(workers):
            if share[k]:
                _serve_phase(trees[k], reqs, p_idx, ph, share[k], out.logs[k])
    for t, lg in zip(trees, out.logs):
        lg.free_list = np.array(list(t.pool.free), np.int32)
        lg.cached_tokens = t.cached_tokens()
        lg.evicted_tokens_total = t.evicted_tokens_total
    return out
