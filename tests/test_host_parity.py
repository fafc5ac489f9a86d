"""The native host library (C++ pool, radix tree, scheduler) against the oracle.

Slot lists, matched lengths, admission order, decode slots, duplicate counts,
the final free list and eviction totals must be bit-identical: both follow the
same reading of the pages (page "49 · RadixAttention, eviction và cache
churn", §2, §4, §5), but share no code. Runs on the CPU (no GPU calls).
"""
import random
import re
import os

import numpy as np
import pytest

from oracle.episode import run_episode
from prefix_shared_kv_radix_amd import _lib
from prefix_shared_kv_radix_amd.runner import Engine
from workloads import (Phase, Workload, _req, agent_branch, chat_decode, chat_tree, config,
                       cyclic_stream, few_shot, gqa128_shape, mla_groups, tiny_shape)


def _compare(w):
    ref = run_episode(w)
    got = Engine(w).run()
    assert len(ref.rounds) == len(got.rounds)
    for r, g in zip(ref.rounds, got.rounds):
        assert r.phase == g.phase
        assert [a.rid for a in r.admissions] == [a.rid for a in g.admissions]
        for a, b in zip(r.admissions, g.admissions):
            assert a.prefix_len == b.prefix_len and a.prompt_len == b.prompt_len, a.rid
            np.testing.assert_array_equal(a.row, b.row)
        np.testing.assert_array_equal(r.decode_slots, g.decode_slots)
        np.testing.assert_array_equal(r.already_cached, g.already_cached)
    np.testing.assert_array_equal(ref.free_list, got.free_list)
    assert ref.cached_tokens == got.stats.cached_tokens
    assert ref.evicted_tokens_total == got.stats.evicted_tokens_total
    assert ref.hits() == got.hits()
    return ref, got


WORKLOADS = {
    "tiny": lambda: config(1),
    "few_shot_small": lambda: few_shot(2, gqa128_shape(), 300, 24, 37, 9),
    "few_shot_full": lambda: config(2),
    "chat_tree_full": lambda: config(3, "A"),
    "chat_tree_tight": lambda: chat_tree(13, tiny_shape(), 12, 6, 5, 40, 0.4),
    "chat_decode_small": lambda: chat_decode(3, tiny_shape(), 12, 100, 600, 16, 64, 5, batch_limit=7),
    "agent_small": lambda: agent_branch(4, tiny_shape(), 3, 100, 4, 30, 3, 7),
    "agent_full": lambda: config(4),
    "cyclic": lambda: config(4, "cyclic"),
    "grouped": lambda: config(4, "grouped"),
    "cyclic_lpf": lambda: config(4, "cyclic_lpf"),
    "mla_small": lambda: mla_groups(5, "bf16", 3, 50, 6, 40, 4, q_rows=64),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_episode_bit_exact(name):
    _compare(WORKLOADS[name]())


def test_churn_numbers_through_native_tree():
    """0/10 cyclic, 5/10 grouped, 5/10 longest-prefix-first (page 4 §6)."""
    assert Engine(config(4, "cyclic")).run().hits()[0] == 0
    assert Engine(config(4, "grouped")).run().hits()[0] == 5
    assert Engine(config(4, "cyclic_lpf")).run().hits()[0] == 5


@pytest.mark.parametrize("seed", range(40))
def test_random_traces_with_tiny_pools(seed):
    """Random prompts over a 3-token alphabet, tiny pools, mixed policies and batch
    limits, with decode steps: heavy splitting and eviction."""
    rng = random.Random(seed)
    n = rng.randint(4, 30)
    reqs = []
    for i in range(n):
        L = rng.randint(1, 9)
        toks = np.array([rng.randint(0, 2) for _ in range(L)], np.int32)
        outs = np.array([rng.randint(0, 2) for _ in range(3)], np.int32)
        reqs.append(_req(i, toks, np.arange(L) + 100 * i, outs, np.arange(3) + 100 * i + 50))
    phases, i = [], 0
    while i < n:
        k = rng.randint(1, 6)
        phases.append(Phase(list(range(i, min(n, i + k))), rng.choice(["fcfs", "lpf"]),
                            rng.randint(1, 4), rng.randint(0, 3), "host"))
        i += k
    pool = rng.randint(16, 40)
    w = Workload("fuzz", seed, tiny_shape(), pool, reqs, phases, 1, 1, 1)
    try:
        ref = run_episode(w)
    except RuntimeError:
        with pytest.raises(RuntimeError):
            Engine(w).run()
        return
    _compare(w)


# ------------------------------------------------------------ ABI behaviour
def test_pool_fifo_errors_and_atomicity():
    p = _lib.KVPool(6)
    np.testing.assert_array_equal(p.alloc(3), [0, 1, 2])
    p.free([1, 0])
    np.testing.assert_array_equal(p.free_list(), [3, 4, 5, 1, 0])
    for bad in ([3], [6], [-1], [2, 2]):
        with pytest.raises(_lib.RadixError) as e:
            p.free(bad)
        assert e.value.status == _lib.E_INVAL
    np.testing.assert_array_equal(p.free_list(), [3, 4, 5, 1, 0])   # unchanged
    with pytest.raises(_lib.NoMemory):
        p.alloc(6)
    assert p.num_free() == 5


def test_tree_nomem_leaves_state_unchanged():
    p = _lib.KVPool(10)
    t = _lib.RadixTree(p)
    m, row, node = t.admit(np.arange(6))
    before = (p.free_list().tolist(), t.stats().tick)
    with pytest.raises(_lib.NoMemory):
        t.alloc(5)
    assert (p.free_list().tolist(), t.stats().tick) == before
    with pytest.raises(_lib.NoMemory):
        t.admit(np.arange(100, 111))       # 11 tokens > 10 slots
    t.finish(np.arange(6), row, m, node)
    assert len(t.alloc(10)) == 10          # everything evictable now


@pytest.mark.parametrize("seed", range(6))
def test_pinned_and_evictable_tokens_match_oracle(seed):
    """Tree statistics while requests are running: pinned tokens (on nodes with a
    nonzero reference count) and evictable tokens equal the oracle's sums over its
    nodes, after every admit and finish of a random interleaving."""
    from oracle import radix as O
    rng = random.Random(seed)
    p = _lib.KVPool(400)
    t = _lib.RadixTree(p)
    op_ = O.SlotPool(400)
    ot = O.RadixTree(op_)
    running = []
    for _ in range(60):
        if running and (rng.random() < 0.45 or len(running) > 6):
            (toks, row, m, node), (orow, om, onode) = running.pop(rng.randrange(len(running)))
            t.finish(toks, row, m, node)
            c = ot.insert(toks, orow)
            op_.release(orow[om:c])
            ot.unlock(onode)
        else:
            toks = np.array([rng.randint(0, 2) for _ in range(rng.randint(1, 12))], np.int32)
            try:
                m, row, node = t.admit(toks)
            except _lib.NoMemory:
                continue
            om, oslots, onode = ot.match(toks)
            ot.lock(onode)
            new = ot.alloc(len(toks) - om)
            assert new is not None
            orow = list(oslots) + list(new)
            assert m == om and row.tolist() == orow
            running.append(((toks, row, m, node), (orow, om, onode)))
        st = t.stats()
        pinned = sum(len(n.key) for n in ot.nodes() if n.lock > 0)
        assert st.pinned_tokens == pinned
        assert st.evictable_tokens == ot.evictable_tokens()
        assert st.cached_tokens == ot.cached_tokens()


def test_unlock_below_zero_and_bad_handles():
    p = _lib.KVPool(10)
    t = _lib.RadixTree(p)
    m, row, node = t.admit(np.arange(3))
    t.finish(np.arange(3), row, m, node)
    m, row, node = t.admit(np.arange(5))        # matches 3 tokens: pins a real node
    assert m == 3 and node != 0
    t.finish(np.arange(5), row, m, node)
    with pytest.raises(_lib.RadixError):
        t.unlock(node)
    with pytest.raises(_lib.RadixError):
        t.lock(12345)


def test_decode_plan_matches_tree_structure():
    """Shared segments follow the radix nodes shared by running requests."""
    w = agent_branch(4, tiny_shape(), 3, 40, 4, 10, 3, 2)
    eng = Engine(w, use_plan=True)
    log = eng.run()
    rnd = log.rounds[-1]
    plan = rnd.plan
    # three roots x 4 branches x 3 forks: root segments (12 members) then branch segments (3)
    assert plan.num_segments == 3 + 12
    sizes = sorted(np.diff(plan.seg_member_off).tolist())
    assert sizes == [3] * 12 + [12] * 3
    assert set(plan.req_num_shared.tolist()) == {2}
    assert set(plan.req_private_start.tolist()) == {50}
    for s in range(plan.num_segments):
        mem = plan.seg_members[plan.seg_member_off[s]:plan.seg_member_off[s + 1]]
        rows = [rnd.admissions[b].row[plan.seg_start[s]:plan.seg_end[s]] for b in mem]
        for r in rows[1:]:
            np.testing.assert_array_equal(r, rows[0])   # members share the slots
        np.testing.assert_array_equal(rnd.admissions[plan.seg_row[s]].row[plan.seg_start[s]:plan.seg_end[s]],
                                      rows[0])


def _random_admissions(seed):
    """A small tree of cached prompts and a batch admitted on it (tree, pool, admissions)."""
    rng = random.Random(seed)
    p = _lib.KVPool(4000)
    t = _lib.RadixTree(p)
    base = [[rng.randint(0, 2) for _ in range(rng.randint(1, 6))] for _ in range(4)]
    for s in base:
        m, row, node = t.admit(s)
        t.finish(s, row, m, node)
    prompts = []
    for _ in range(rng.randint(2, 10)):
        b = rng.choice(base)
        prompts.append(b[:rng.randint(0, len(b))] + [rng.randint(0, 2) for _ in range(rng.randint(0, 3))])
    return t, p, [t.admit(pr) for pr in prompts]


def test_decode_plan_brute_force():
    """Random batches: for each pair of requests, the shared segments they have in
    common cover exactly the prefix of identical slots up to the shallower private start."""
    for seed in range(20):
        t, p, adm = _random_admissions(seed)
        plan = t.decode_plan([a[2] for a in adm])
        for i in range(len(adm)):
            segs = [s for s in range(plan.num_segments)
                    if i in plan.seg_members[plan.seg_member_off[s]:plan.seg_member_off[s + 1]]]
            cover = sorted((plan.seg_start[s], plan.seg_end[s]) for s in segs)
            pos = 0
            for a0, a1 in cover:
                assert a0 == pos
                pos = a1
            assert pos == plan.req_private_start[i] <= adm[i][0]
            for s in segs:
                mem = plan.seg_members[plan.seg_member_off[s]:plan.seg_member_off[s + 1]]
                assert len(mem) >= 2
                for j in mem:
                    np.testing.assert_array_equal(adm[j][1][plan.seg_start[s]:plan.seg_end[s]],
                                                  adm[i][1][plan.seg_start[s]:plan.seg_end[s]])


def test_decode_plan_request_order_groups_root_segments():
    """Random batches (members of a prefix in any batch order): req_order is a
    permutation of the batch that lists the members of each segment starting at the
    root together (a request has at most one), and the requests with no shared
    segment last, in batch order."""
    for seed in range(40):
        t, p, adm = _random_admissions(seed)
        plan = t.decode_plan([a[2] for a in adm])
        order = np.asarray(plan.req_order).tolist()
        B = len(adm)
        assert sorted(order) == list(range(B))
        at = {b: i for i, b in enumerate(order)}
        shared = set()
        for s_ in range(plan.num_segments):
            mem = plan.seg_members[plan.seg_member_off[s_]:plan.seg_member_off[s_ + 1]].tolist()
            shared.update(mem)
            if plan.seg_start[s_] == 0:
                idx = sorted(at[b] for b in mem)
                assert idx == list(range(idx[0], idx[0] + len(idx)))
        rest = [b for b in order if b not in shared]
        assert order[len(order) - len(rest):] == sorted(rest)


def test_mla_plan_keeps_each_group_on_one_xcd():
    """Config 5 (MLA, batch 256, groups of 32 requests sharing a 2048-token prefix): the
    MLA decode launch gives request-order positions [x * ceil(B / 8), (x + 1) * ceil(B / 8))
    to XCD x (one key split per request at this batch), so with the plan's req_order
    (the members of each shared segment listed together) every group's prefix rows are
    read through one XCD's L2."""
    w = config(5, "bf16")
    plans = [r.plan for r in Engine(w).run().rounds if r.plan is not None]
    assert plans
    for plan in plans:
        order = np.asarray(plan.req_order)
        B = len(order)
        assert sorted(order.tolist()) == list(range(B))
        at = np.empty(B, np.int64)
        at[order] = np.arange(B)
        per = -(-B // 8)
        assert plan.num_segments == 8
        for s_ in range(plan.num_segments):
            mem = np.asarray(plan.seg_members[plan.seg_member_off[s_]:plan.seg_member_off[s_ + 1]])
            assert len(mem) == 32
            assert len(set((at[mem] // per).tolist())) == 1


def test_decode_plan_key_chunks():
    """Key chunks: the segments do not depend on split_keys; segment s gets
    ceil(len / split_keys) chunks (1 when split_keys <= 0 or len <= split_keys); each
    request's partial indices (segments in path order, a segment's chunks consecutive)
    tile 0 .. req_num_parts-1 exactly; the host counts agree with the arrays."""
    checked = 0
    for seed in range(30):
        t, p, adm = _random_admissions(seed)
        nodes = [a[2] for a in adm]
        ref = t.decode_plan(nodes)
        for sk in (0, -3, 1, 2, 3, 5):
            plan = t.decode_plan(nodes, 2, sk)
            for f in ("seg_row", "seg_start", "seg_end", "seg_member_off", "seg_members",
                      "seg_member_slot", "req_num_shared", "req_private_start", "req_order"):
                np.testing.assert_array_equal(getattr(plan, f), getattr(ref, f))
            lens = plan.seg_end - plan.seg_start
            want = np.array([1 if sk <= 0 or n <= sk else -(-n // sk) for n in lens], np.int64)
            assert plan.seg_split_off[0] == 0
            np.testing.assert_array_equal(np.diff(plan.seg_split_off), want)
            assert plan.num_seg_items == int(want.sum())
            assert plan.max_seg_splits == (int(want.max()) if len(want) else 0)
            # chunk records: the chunks of segment s tile [start, end) in order, each at
            # most one rounded-up share long, with the segment's members and row
            rec = plan.seg_items.reshape(-1, 8)
            assert len(rec) == plan.num_seg_items
            for s_ in range(plan.num_segments):
                k0, k1 = plan.seg_split_off[s_], plan.seg_split_off[s_ + 1]
                n_ = int(lens[s_])
                share = -(-(-(-n_ // (k1 - k0))) // 64) * 64
                pos = plan.seg_start[s_]
                for k in range(k0, k1):
                    r = rec[k]
                    assert r[0] == pos and pos <= r[1] <= plan.seg_end[s_] and r[1] - r[0] <= share
                    assert r[1] - r[0] == min(share, plan.seg_end[s_] - pos)
                    pos = r[1]
                    assert (r[2], r[3], r[4], r[5], r[6]) == (
                        plan.seg_member_off[s_], plan.seg_member_off[s_ + 1] - plan.seg_member_off[s_],
                        plan.seg_row[s_], s_, k - k0)
                assert pos == plan.seg_end[s_]
            for i in range(len(adm)):
                owned = []   # (rank, first part, chunks) of request i's segments
                for s_ in range(plan.num_segments):
                    lo, hi = plan.seg_member_off[s_], plan.seg_member_off[s_ + 1]
                    for e in range(lo, hi):
                        if plan.seg_members[e] == i:
                            owned.append((plan.seg_member_slot[e], plan.seg_member_part[e], want[s_]))
                owned.sort()
                assert [o[0] for o in owned] == list(range(len(owned)))
                nxt = 0
                for _, first, n in owned:
                    assert first == nxt
                    nxt += n
                assert plan.req_num_parts[i] == nxt
                checked += len(owned)
            assert plan.max_parts == (int(plan.req_num_parts.max()) if len(adm) else 0)
    assert checked > 50


def test_segment_chunk_policy():
    """The runner cuts a round's shared segments at half the longest one (1024..2048
    keys per chunk): the few-shot 2048-token prefix and the agent 4096-token roots get
    two chunks each, the 512-token branches stay whole."""
    from prefix_shared_kv_radix_amd.runner import seg_split_keys
    assert [seg_split_keys(n) for n in (0, 1024, 1025, 1500, 2048, 4096, 8192)] == \
        [0, 0, 1024, 1024, 1024, 2048, 2048]
    for n, chunks in ((2, {2048: 2}), (4, {4096: 2, 512: 1})):
        log = Engine(config(n)).run()
        plans = [r.plan for r in log.rounds if r.plan is not None]
        assert plans
        for plan in plans:
            lens = plan.seg_end - plan.seg_start
            splits = np.diff(plan.seg_split_off)
            for ln, k in zip(lens, splits):
                assert chunks[int(ln)] == int(k), (n, ln, k)


def test_decode_workspace_covers_late_private_chunks():
    """A bf16 decode step with a plan and one private chunk per request reads the
    private keys of its last tenth of requests (launch order) in two chunks, once
    the private tails reach 64 keys: its workspace then holds two private partials per
    request, as with num_splits = 2. fp32 steps, steps without a plan and shorter tails
    keep one chunk, as do batches under 10 (no request in the last tenth)."""
    def plan(min_private_start):
        return _lib.DecodePlan(1, 256, *([None] * len(_lib._PLAN_ARRAYS)), 256, 1, 2048,
                               min_private_start, 2, 2, 2)
    bf16 = _lib.make_shape(32, 8, 128, 128, "bf16", "bf16", False, 0.088)
    f32 = _lib.make_shape(32, 8, 128, 128, "f32", "f32", False, 0.088)
    ws = _lib.decode_workspace_size
    for batch in (10, 256):   # at least one request in the last tenth
        long_tail = plan(2048)
        assert ws(bf16, batch, 2048 + 256, long_tail, 0) == ws(bf16, batch, 2048 + 256, long_tail, 2)
        assert ws(bf16, batch, 2048 + 256, long_tail, 0) > ws(bf16, batch, 2048 + 256, long_tail, 1)
        assert ws(bf16, batch, 2048 + 63, long_tail, 0) == ws(bf16, batch, 2048 + 63, long_tail, 1)
        assert ws(f32, batch, 2048 + 256, long_tail, 0) == ws(f32, batch, 2048 + 256, long_tail, 1)
    assert ws(bf16, 256, 1000, None, 0) == ws(bf16, 256, 1000, None, 1)
    assert ws(bf16, 9, 2048 + 256, plan(2048), 0) == ws(bf16, 9, 2048 + 256, plan(2048), 1)


def test_library_exports_every_declared_symbol():
    """Every function declared in include/*.h is exported by the built library."""
    import ctypes
    hdr_dir = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
    names = set()
    for f in os.listdir(hdr_dir):
        if f.endswith(".h"):
            text = open(os.path.join(hdr_dir, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(radix_[a-z0-9_]+)\s*\(", text))
    assert len(names) > 20
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_lib.exported_symbols()) <= names
