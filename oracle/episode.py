"""Oracle: run a workload's request script through the oracle tree.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Request lifecycle (page "49 · RadixAttention, eviction và cache churn", §2 and
§4; SGLang overview, nine-step example):
  admit  : match the prompt (longest cached prefix, m tokens), pin the matched
           path, take len - m new slots (evicting when short). If the slots
           cannot be had, unpin and leave the request waiting; admission for
           the round stops there.
  decode : every step takes one slot per running request, in admission order.
  finish : insert prompt + generated tokens with the request's slots; slots of
           tokens some other request inserted meanwhile are given back; unpin.
A request whose prompt is fully cached has nothing to extend (E = 0).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .radix import RadixTree, SlotPool, schedule_order


@dataclass
class Admission:
    rid: int
    prefix_len: int            # matched tokens m
    prompt_len: int
    row: np.ndarray            # int32 slots of the prompt positions (m cached + new)


@dataclass
class Round:
    phase: int
    admissions: List[Admission]
    decode_slots: np.ndarray   # int32 [n_decode, batch], admission order
    already_cached: np.ndarray  # int64 [batch] from insert at finish


@dataclass
class EpisodeLog:
    rounds: List[Round] = field(default_factory=list)
    free_list: np.ndarray = None
    cached_tokens: int = 0
    evicted_tokens_total: int = 0

    def hits(self):
        """(requests fully matched, matched tokens, prompt tokens)."""
        req = sum(1 for r in self.rounds for a in r.admissions if a.prefix_len == a.prompt_len)
        mt = sum(a.prefix_len for r in self.rounds for a in r.admissions)
        pt = sum(a.prompt_len for r in self.rounds for a in r.admissions)
        return req, mt, pt


def run_episode(workload) -> EpisodeLog:
    pool = SlotPool(workload.pool_slots)
    tree = RadixTree(pool)
    log = EpisodeLog()
    reqs = workload.requests
    for p_idx, ph in enumerate(workload.phases):
        waiting = list(ph.rids)
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
            cached_counts = np.zeros(len(admitted), np.int64)
            for b, (a, node) in enumerate(zip(admitted, nodes)):
                r = reqs[a.rid]
                full_tok = np.concatenate([r.tokens, r.out_tokens[:ph.n_decode]])
                full_row = np.concatenate([a.row, dec[:, b]]).astype(np.int32)
                c = tree.insert(full_tok, full_row)
                cached_counts[b] = c
                if c > a.prefix_len:
                    pool.release(full_row[a.prefix_len:c])
                tree.unlock(node)
            log.rounds.append(Round(p_idx, admitted, dec, cached_counts))
    log.free_list = np.asarray(pool.free, np.int32)
    log.cached_tokens = tree.cached_tokens()
    log.evicted_tokens_total = tree.evicted_tokens_total
    return log
