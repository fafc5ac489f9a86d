"""Oracle: slot pool, radix tree, eviction and scheduling, in plain Python.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module;
only tests, the smoke check and the bench's CPU baseline do.

The tree caches K/V slots for token sequences so later requests reuse them.
It follows the page "49 · RadixAttention, eviction và cache churn":
  §2  every edge holds a run of tokens plus the K/V slots of those tokens; a
      lookup walks token by token until the tokens differ, and where it
      diverges inside an edge, that edge splits into a shared part and two
      branches; a finished request's whole path (outputs included) stays.
  §4  cache and running requests share one slot pool; running requests pin
      their path with a reference count and only count-0 nodes may go;
      leaves go first, least recently used first; a node whose children are
      all gone becomes a leaf and may go later.
  §5  longest-cached-prefix-first ordering.
and the SGLang overview article (unite.ai), section "SGLang: Mô Hình Lập
Trình và Phương Pháp": an LRU cache of KV in a radix tree used for matching,
insertion and eviction (nine-step example).

Where the pages are silent the oracle takes these readings:
  * free list: FIFO, initially 0..N-1 ascending; freed slots are appended in
    the order given;
  * clock: one logical tick per mutating match/insert; peek does not tick;
    a split's upper node gets the current tick, the lower keeps its own;
  * eviction removes whole leaf nodes (it may free more than asked); among
    candidates the smallest (tick, root-to-node token path) goes first;
  * allocation is all-or-nothing: if free + evictable < n nothing changes.
"""
from __future__ import annotations

import heapq
import itertools
from collections import deque
from typing import List, Optional, Tuple

import numpy as np


class PoolError(ValueError):
    pass


class SlotPool:
    """A FIFO free list over slot indices 0..num_slots-1."""

    def __init__(self, num_slots: int):
        if num_slots < 0:
            raise PoolError("negative pool size")
        self.num_slots = int(num_slots)
        self.free = deque(range(self.num_slots))
        self.is_free = np.ones(self.num_slots, dtype=bool)

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, n: int) -> Optional[List[int]]:
        if n < 0:
            raise PoolError("negative count")
        if len(self.free) < n:
            return None
        out = [self.free.popleft() for _ in range(n)]
        self.is_free[out] = False
        return out

    def release(self, slots) -> None:
        slots = [int(s) for s in slots]
        seen = set()
        for s in slots:
            if s < 0 or s >= self.num_slots or self.is_free[s] or s in seen:
                raise PoolError(f"bad free of slot {s}")
            seen.add(s)
        for s in slots:
            self.is_free[s] = True
            self.free.append(s)


class Node:
    __slots__ = ("key", "value", "children", "parent", "lock", "tick")

    def __init__(self, key, value, parent, lock, tick):
        self.key = key          # np.int32 token ids on the edge into this node
        self.value = value      # np.int32 slots of those tokens
        self.children = {}      # first token -> child
        self.parent = parent
        self.lock = lock
        self.tick = tick

    def path(self) -> Tuple[int, ...]:
        parts = []
        n = self
        while n.parent is not None:
            parts.append(n.key)
            n = n.parent
        if not parts:
            return ()
        return tuple(int(t) for t in np.concatenate(parts[::-1]))


def lcp(a: np.ndarray, b: np.ndarray) -> int:
    """Length of the longest common prefix of two token arrays."""
    n = min(len(a), len(b))
    if n == 0:
        return 0
    diff = np.nonzero(a[:n] != b[:n])[0]
    return int(diff[0]) if len(diff) else n


class _EvictKey:
    """Heap key: (tick, path); the path is only built when ticks tie."""
    __slots__ = ("node",)

    def __init__(self, node):
        self.node = node

    def __lt__(self, other):
        return self.node.path() < other.node.path()

    def __eq__(self, other):
        return self.node is other.node


class RadixTree:
    def __init__(self, pool: SlotPool):
        self.pool = pool
        self.root = Node(np.zeros(0, np.int32), np.zeros(0, np.int32), None, 0, 0)
        self.tick = 0
        self.evicted_tokens_total = 0
        self.evict_log: List[Tuple[int, int]] = []   # (tick, token count) per evicted node

    # ---- walking -------------------------------------------------------
    def _split(self, c: Node, k: int) -> Node:
        upper = Node(c.key[:k].copy(), c.value[:k].copy(), c.parent, c.lock, self.tick)
        c.parent.children[int(c.key[0])] = upper
        c.key = c.key[k:].copy()
        c.value = c.value[k:].copy()
        c.parent = upper
        upper.children[int(c.key[0])] = c
        return upper

    def _walk(self, tokens: np.ndarray):
        """Walk from the root, splitting a partially matched edge and refreshing ticks."""
        node, i, slots = self.root, 0, []
        n = len(tokens)
        while i < n:
            c = node.children.get(int(tokens[i]))
            if c is None:
                break
            k = lcp(c.key, tokens[i:])
            if k < len(c.key):
                c = self._split(c, k)
            c.tick = self.tick
            slots.append(c.value)
            i += k
            node = c
        matched = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
        return i, matched, node

    def match(self, tokens) -> Tuple[int, np.ndarray, Node]:
        """Longest cached prefix: (matched length, its slots, last node on the path)."""
        tokens = np.asarray(tokens, dtype=np.int32)
        self.tick += 1
        return self._walk(tokens)

    def peek(self, tokens) -> int:
        """Matched length without splitting or refreshing anything (may end mid-edge)."""
        tokens = np.asarray(tokens, dtype=np.int32)
        node, i, n = self.root, 0, len(tokens)
        while i < n:
            c = node.children.get(int(tokens[i]))
            if c is None:
                break
            k = lcp(c.key, tokens[i:])
            i += k
            if k < len(c.key):
                break
            node = c
        return i

    def insert(self, tokens, slots) -> int:
        """Insert a finished sequence; returns how many leading tokens were already cached."""
        tokens = np.asarray(tokens, dtype=np.int32)
        slots = np.asarray(slots, dtype=np.int32)
        if len(tokens) != len(slots):
            raise ValueError("tokens and slots differ in length")
        self.tick += 1
        i, _, node = self._walk(tokens)
        if i < len(tokens):
            leaf = Node(tokens[i:].copy(), slots[i:].copy(), node, 0, self.tick)
            node.children[int(tokens[i])] = leaf
        return i

    # ---- pinning ---------------------------------------------------------
    def lock(self, node: Node) -> None:
        while node is not self.root:
            node.lock += 1
            node = node.parent

    def unlock(self, node: Node) -> None:
        while node is not self.root:
            if node.lock <= 0:
                raise ValueError("unlock of an unpinned node")
            node.lock -= 1
            node = node.parent

    # ---- eviction ----------------------------------------------------------
    def nodes(self):
        stack = list(self.root.children.values())
        while stack:
            n = stack.pop()
            yield n
            stack.extend(n.children.values())

    def evictable_tokens(self) -> int:
        return sum(len(n.key) for n in self.nodes() if n.lock == 0)

    def cached_tokens(self) -> int:
        return sum(len(n.key) for n in self.nodes())

    def evict(self, need: int) -> int:
        """Evict unpinned leaves, least recently used first, until ``need`` slots are freed."""
        counter = itertools.count()
        heap = [(n.tick, _EvictKey(n), next(counter), n)
                for n in self.nodes() if not n.children and n.lock == 0]
        heapq.heapify(heap)
        freed = 0
        while freed < need and heap:
            _, _, _, n = heapq.heappop(heap)
            self.pool.release(n.value)
            freed += len(n.value)
            self.evicted_tokens_total += len(n.value)
            self.evict_log.append((n.tick, len(n.value)))
            parent = n.parent
            del parent.children[int(n.key[0])]
            n.parent = None
            if parent is not self.root and not parent.children and parent.lock == 0:
                heapq.heappush(heap, (parent.tick, _EvictKey(parent), next(counter), parent))
        return freed

    def alloc(self, n: int) -> Optional[List[int]]:
        """Take n slots, evicting leaf-first LRU when short; None (no change) if impossible."""
        if self.pool.num_free() >= n:
            return self.pool.alloc(n)
        if self.pool.num_free() + self.evictable_tokens() < n:
            return None
        self.evict(n - self.pool.num_free())
        return self.pool.alloc(n)


def schedule_order(tree: RadixTree, prompts, policy: str) -> List[int]:
    """Admission order: 'fcfs' keeps arrival order; 'lpf' sorts by the longest cached
    prefix, longest first, keeping arrival order among equals (page 4 §5)."""
    n = len(prompts)
    if policy == "fcfs":
        return list(range(n))
    if policy == "lpf":
        lens = [tree.peek(p) for p in prompts]
        return sorted(range(n), key=lambda i: -lens[i])
    raise ValueError(policy)
