"""Oracle: the same request scripts through a block-granular hash-chain prefix cache.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The page "49 · RadixAttention, eviction và cache churn", §3, sets RadixAttention's
token-level radix tree beside prefix caching keyed by a chain of block hashes
(vLLM): both reuse any common prefix automatically, share blocks by reference
count and evict least recently used first, but the hash chain matches in steps of
a 16-token block while the radix tree matches token by token. This module replays
a workload through such a block cache so the two can be compared on the same
traces (reused tokens, hit rates).

Readings where the page is silent (the comparison only needs the matching
granularity and the eviction rule):
  * block size 16; the pool holds pool_slots // 16 blocks; a FIFO free list of
    block indices, initially ascending (as the slot pool);
  * a block's identity is its 16 tokens together with the identity of the block
    before it (the chain hash, here kept exact: no collisions);
  * a prompt of n tokens matches its longest run of leading full blocks that are
    cached; the partial last block is never shared;
  * admission: match, pin the matched blocks, take ceil(n/16) - matched new blocks
    (evicting when short; all or nothing, as for the tree); decode takes a new block
    whenever the sequence length reaches a multiple of 16;
  * finish: the full blocks of prompt + outputs not cached yet become cached (a
    block some other request cached meanwhile is given back), the partial last
    block is given back, the pins are released;
  * clock: one tick per admission match and per finish; a touched block takes the
    tick; eviction takes the unpinned cached block with the smallest tick, the
    deeper block first on equal ticks (so a chain's tail goes before its head);
  * scheduling: FCFS, or longest cached prefix first with the block match length.
"""
from __future__ import annotations

import heapq
from collections import deque
from dataclasses import dataclass, field
from typing import List

import numpy as np

BLOCK = 16


@dataclass
class _Block:
    index: int        # pool block index
    depth: int        # position of the block in its chain (0 = first)
    ref: int = 0
    tick: int = 0


class BlockHashCache:
    def __init__(self, num_slots: int, block: int = BLOCK):
        self.block = block
        self.num_blocks = num_slots // block
        self.free = deque(range(self.num_blocks))
        self.ids = {}       # (parent chain id, block tokens) -> chain id
        self.cached = {}    # chain id -> _Block
        self.tick = 0
        self.evicted_blocks = 0

    # ---- identities ------------------------------------------------------
    def chain_ids(self, tokens, create: bool):
        """Chain ids of the full blocks of `tokens`; stops at the first unknown block
        unless `create`."""
        out, parent = [], -1
        b = self.block
        tokens = np.asarray(tokens, dtype=np.int32)
        for j in range(len(tokens) // b):
            key = (parent, tokens[j * b:(j + 1) * b].tobytes())   # the block's 16 token ids
            cid = self.ids.get(key)
            if cid is None:
                if not create:
                    break
                cid = len(self.ids)
                self.ids[key] = cid
            out.append(cid)
            parent = cid
        return out

    # ---- lookup ----------------------------------------------------------
    def peek(self, tokens) -> int:
        """Reused tokens: leading full blocks that are cached, without touching them."""
        n = 0
        for cid in self.chain_ids(tokens, False):
            if cid not in self.cached:
                break
            n += 1
        return n * self.block

    def match(self, tokens):
        """(matched blocks' chain ids) of the longest cached run of leading blocks; the
        matched blocks take the new tick."""
        self.tick += 1
        got = []
        for cid in self.chain_ids(tokens, False):
            blk = self.cached.get(cid)
            if blk is None:
                break
            blk.tick = self.tick
            got.append(cid)
        return got

    # ---- pool ------------------------------------------------------------
    def evictable(self) -> int:
        return sum(1 for blk in self.cached.values() if blk.ref == 0)

    def alloc(self, n: int):
        """n free block indices, evicting unpinned cached blocks least recently used
        first (deeper first on equal ticks); None (nothing changed) if impossible."""
        if len(self.free) + self.evictable() < n:
            return None
        if len(self.free) < n:
            heap = [(blk.tick, -blk.depth, cid) for cid, blk in self.cached.items() if blk.ref == 0]
            heapq.heapify(heap)
            while len(self.free) < n:
                _, _, cid = heapq.heappop(heap)
                self.free.append(self.cached.pop(cid).index)
                self.evicted_blocks += 1
        return [self.free.popleft() for _ in range(n)]

    def release(self, blocks) -> None:
        self.free.extend(int(x) for x in blocks)


@dataclass
class BlockAdmission:
    rid: int
    reused: int            # tokens served from cached blocks
    prompt_len: int
    matched: List[int]     # chain ids of the matched blocks (pinned)
    own: List[int]         # pool blocks this request took


@dataclass
class BlockEpisodeLog:
    admissions: List[BlockAdmission] = field(default_factory=list)
    evicted_blocks: int = 0
    num_blocks: int = 0
    free_blocks: int = 0       # at the end of the episode
    cached_blocks: int = 0     # at the end of the episode

    def hits(self):
        """(requests whose whole prompt was reused, reused tokens, prompt tokens)."""
        req = sum(1 for a in self.admissions if a.reused == a.prompt_len)
        return req, sum(a.reused for a in self.admissions), sum(a.prompt_len for a in self.admissions)


def _order(cache: BlockHashCache, prompts, policy: str) -> List[int]:
    if policy == "fcfs":
        return list(range(len(prompts)))
    if policy == "lpf":
        lens = [cache.peek(p) for p in prompts]
        return sorted(range(len(prompts)), key=lambda i: -lens[i])   # stable: ties keep order
    raise ValueError(policy)


def run_block_episode(workload, block: int = BLOCK) -> BlockEpisodeLog:
    """The workload's rounds (same phases, policies and batch limits as the radix
    episode) through a block-hash cache."""
    cache = BlockHashCache(workload.pool_slots, block)
    log = BlockEpisodeLog()
    reqs = workload.requests
    for ph in workload.phases:
        waiting = list(ph.rids)
        while waiting:
            order = _order(cache, [reqs[r].tokens for r in waiting], ph.policy)
            waiting = [waiting[i] for i in order]
            admitted = []
            for rid in waiting:
                if len(admitted) >= ph.batch_limit:
                    break
                toks = reqs[rid].tokens
                matched = cache.match(toks)
                for cid in matched:
                    cache.cached[cid].ref += 1
                need = -(-len(toks) // block) - len(matched)
                own = cache.alloc(need)
                if own is None:
                    for cid in matched:
                        cache.cached[cid].ref -= 1
                    break
                admitted.append(BlockAdmission(rid, len(matched) * block, len(toks), matched, own))
            if not admitted:
                raise RuntimeError(f"request {waiting[0]} cannot be admitted into an idle pool")
            taken = {a.rid for a in admitted}
            waiting = [r for r in waiting if r not in taken]
            for s in range(ph.n_decode):
                for a in admitted:
                    if (a.prompt_len + s) % block == 0:   # the next token opens a new block
                        got = cache.alloc(1)
                        if got is None:
                            raise RuntimeError("pool exhausted during decode")
                        a.own.extend(got)
            for a in admitted:
                r = reqs[a.rid]
                seq = np.concatenate([r.tokens, r.out_tokens[:ph.n_decode]])
                cache.tick += 1
                ids = cache.chain_ids(seq, True)
                nm = len(a.matched)
                for j, cid in enumerate(ids):
                    if j < nm:
                        cache.cached[cid].tick = cache.tick
                        continue
                    blk_index = a.own[j - nm]
                    if cid in cache.cached:      # cached by another request meanwhile
                        cache.cached[cid].tick = cache.tick
                        cache.release([blk_index])
                    else:
                        cache.cached[cid] = _Block(blk_index, j, 0, cache.tick)
                cache.release(a.own[len(ids) - nm:])     # the partial last block
                for cid in a.matched:
                    cache.cached[cid].ref -= 1
                log.admissions.append(a)
    log.evicted_blocks = cache.evicted_blocks
    log.num_blocks = cache.num_blocks
    log.free_blocks = len(cache.free)
    log.cached_blocks = len(cache.cached)
    return log
