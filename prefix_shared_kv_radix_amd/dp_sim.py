"""Data-parallel serving simulated on the host: several workers, each with its own slot
pool and radix tree (one GPU each), and a router in front of them.

The SGLang feature article spreads batches over independent data-parallel attention
workers so that no KV is stored twice (§一) and names a cache-aware load balancer
(§五, heading only). Here each phase's requests arrive together; the router
(radix_route, native) assigns them one by one against the workers' trees as they
stand at the start of the phase, counting the requests it has queued on each
worker as that worker's load; then every worker serves its share of the phase in
rounds exactly as a single GPU does (runner.Engine.run_phase: order, admit with
eviction, decode-slot allocation, insert). Nothing runs on a GPU: the point is
where the cached prefixes end up (reuse, recomputation, duplication and balance),
which is host-side state.

Usage: python -m prefix_shared_kv_radix_amd.dp_sim [workers]   (prints one JSON line
per workload and policy)
"""
from __future__ import annotations

import dataclasses
import json
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

from . import _lib
from .runner import Engine, EpisodeLog


@dataclass
class DPResult:
    workers: int
    policy: str
    assignment: Dict[int, Tuple[int, int]] = field(default_factory=dict)  # rid -> (worker, peek)
    logs: List[EpisodeLog] = field(default_factory=list)

    def summary(self, w) -> dict:
        reused = [sum(a.prefix_len for r in lg.rounds for a in r.admissions) for lg in self.logs]
        computed = [sum(a.prompt_len - a.prefix_len for r in lg.rounds for a in r.admissions)
                    for lg in self.logs]
        reqs = [sum(len(r.admissions) for r in lg.rounds) for lg in self.logs]
        prompt = sum(len(w.requests[rid].tokens) for rid in self.assignment)
        mean = float(np.mean(computed)) if computed else 0.0
        return {"workload": w.name, "workers": self.workers, "policy": self.policy,
                "prompt_tokens": prompt, "reused_tokens": int(sum(reused)),
                "evicted_tokens": int(sum(lg.stats.evicted_tokens_total for lg in self.logs)),
                "token_hit_rate": sum(reused) / prompt if prompt else 0.0,
                "computed_tokens": int(sum(computed)),
                "max_worker_computed": int(max(computed)),
                "computed_imbalance": max(computed) / mean if mean else 1.0,
                "requests_per_worker": reqs,
                "cached_tokens_total": int(sum(lg.stats.cached_tokens for lg in self.logs))}


def run_dp(workload, workers: int, policy: str, balance_abs: int = 32,
           balance_rel: float = 1.5, pool_factor: float = 2.0) -> DPResult:
    """Each worker's pool holds pool_factor x the workload's single-GPU pool: a policy
    that scatters a shared prefix makes every worker hold (and recompute) its own copy,
    which the single-GPU sizing does not leave room for."""
    wk = dataclasses.replace(workload, pool_slots=int(workload.pool_slots * pool_factor))
    engines = [Engine(wk) for _ in range(workers)]
    router = _lib.Router([e.tree for e in engines], policy, balance_abs, balance_rel)
    res = DPResult(workers, policy, logs=[EpisodeLog() for _ in range(workers)])
    for p_idx, ph in enumerate(workload.phases):
        loads = np.zeros(workers, np.int64)
        share: List[List[int]] = [[] for _ in range(workers)]
        for rid in ph.rids:
            k, m = router.route(wk.requests[rid].tokens, loads)
            share[k].append(rid)
            loads[k] += 1
            res.assignment[rid] = (k, m)
        for k in range(workers):
            if share[k]:
                engines[k].run_phase(p_idx, ph, share[k], res.logs[k])
    for e, lg in zip(engines, res.logs):
        lg.free_list = e.pool.free_list()
        lg.stats = e.tree.stats()
    return res


def main():
    from workloads import config
    workers = int(sys.argv[1]) if len(sys.argv) > 1 else 8
    for n, v in [(2, ""), (3, "A"), (4, ""), (5, "bf16")]:
        w = config(n, v)
        for policy in ("round_robin", "least_load", "cache_aware"):
            print(json.dumps(run_dp(w, workers, policy).summary(w)), flush=True)


if __name__ == "__main__":
    main()
