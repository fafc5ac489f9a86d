"""Serving loop over a workload script: native tree/scheduler on the host,
HIP kernels on the device.

Request lifecycle (page "49 · RadixAttention, eviction và cache churn", §2, §4,
§5): per round the waiting queue is ordered (FCFS or longest cached prefix
first), requests are admitted until the batch limit or until the pool cannot
supply their new slots (then the rest wait), the admitted batch is extended as
one call, decoded step by step (one new slot per request per step) and
finished (inserted with its outputs, duplicates given back, unpinned).

This module only sequences calls into libradix_attn; all matching, eviction,
ordering, segment planning and attention happen in native code.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

from . import _lib


@dataclass
class Admission:
    rid: int
    prefix_len: int
    prompt_len: int
    row: np.ndarray
    node: int = 0


@dataclass
class RoundLog:
    phase: int
    admissions: List[Admission]
    decode_slots: np.ndarray
    already_cached: np.ndarray
    plan: Optional[_lib.HostPlan] = None


@dataclass
class EpisodeLog:
    rounds: List[RoundLog] = field(default_factory=list)
    free_list: np.ndarray = None
    stats: object = None

    def hits(self):
        req = sum(1 for r in self.rounds for a in r.admissions if a.prefix_len == a.prompt_len)
        mt = sum(a.prefix_len for r in self.rounds for a in r.admissions)
        pt = sum(a.prompt_len for r in self.rounds for a in r.admissions)
        return req, mt, pt


_TORCH_KV = {"f32": "float32", "bf16": "bfloat16", "fp8": "uint8"}

# Shared segments are cut into key chunks in the decode plan, each its own unit of work,
# so that a long shared prefix is not one block's sequential walk: a round's plan cuts
# at half its longest segment, at least SEG_CHUNK_MIN and at most SEG_CHUNK_MAX keys per
# chunk, and keeps segments up to SEG_CHUNK_MIN keys whole. Measured on one MI355X: a
# 2048-key prefix shared by 256 requests and 4096-key roots shared by 32 requests are
# both fastest in two chunks; shorter chunks add more per-chunk work (prologue, partial,
# merge) than they save in chain length.
SEG_CHUNK_MIN, SEG_CHUNK_MAX = 1024, 2048


def seg_split_keys(longest: int) -> int:
    """split_keys for a plan whose longest shared segment has `longest` keys (0: none)."""
    if longest <= SEG_CHUNK_MIN:
        return 0
    return min(SEG_CHUNK_MAX, max(SEG_CHUNK_MIN, (longest + 1) // 2))


def build_decode_plan(tree, nodes, min_members: int = 2, split_keys: Optional[int] = None):
    """The round's shared-segment plan; split_keys None picks it with seg_split_keys."""
    if split_keys is not None:
        return tree.decode_plan(nodes, min_members, split_keys)
    plan = tree.decode_plan(nodes, min_members, 0)
    sk = seg_split_keys(plan.max_seg_len)
    return plan if sk == 0 else tree.decode_plan(nodes, min_members, sk)


class DeviceState:
    """Device buffers for one workload: the K/V pool, slot lists, tables of inputs."""

    def __init__(self, workload, device, max_batch, rtt_stride):
        import torch
        self.torch = torch
        w = workload
        s = w.shape
        self.device = device
        self.shape = _lib.make_shape(s.num_q_heads, s.num_kv_heads, s.head_dim_qk, s.head_dim_v,
                                     s.q_dtype, s.kv_dtype, s.v_is_k_prefix, s.sm_scale)
        kv_t = getattr(torch, _TORCH_KV[s.kv_dtype])
        q_t = getattr(torch, _TORCH_KV[s.q_dtype])
        n = w.pool_slots
        self.k_pool = torch.zeros((n, s.num_kv_heads, s.head_dim_qk), dtype=kv_t, device=device)
        self.v_pool = None if s.v_is_k_prefix else torch.zeros(
            (n, s.num_kv_heads, s.head_dim_v), dtype=kv_t, device=device)
        self.kv_scale = torch.ones(n, dtype=torch.float32, device=device) \
            if s.kv_dtype == "fp8" else None
        self.kv = _lib.make_kv(self.k_pool, self.v_pool, self.kv_scale)
        k_tab, v_tab, sc = w.kv_table()
        self.k_tab = self._upload(k_tab, kv_t)
        self.v_tab = None if v_tab is None else self._upload(v_tab, kv_t)
        self.sc_tab = None if sc is None else torch.from_numpy(sc).to(device)
        self.q_tab = self._upload(w.q_table(), q_t)
        self.q_dtype = q_t
        self.rtt = torch.zeros((max_batch, rtt_stride), dtype=torch.int32, device=device)
        self.rtt_stride = rtt_stride

    def _upload(self, arr, dtype):
        t = self.torch.from_numpy(np.ascontiguousarray(arr))
        if arr.dtype == np.uint16:
            t = t.view(self.torch.int16)
        return t.to(self.device).view(dtype)

    def i32(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.device)

    def rows_of(self, w, kv_ids):
        return self.torch.from_numpy(w.kv_rows(kv_ids)).to(self.device)


class Engine:
    """Runs a workload through the native tree (and, with a device, the kernels)."""

    def __init__(self, workload, device=None, use_plan: bool = True, num_splits: int = 0,
                 on_extend: Optional[Callable] = None, on_decode: Optional[Callable] = None,
                 min_members: int = 2, host_slots: bool = False,
                 split_keys: Optional[int] = None, noalloc: bool = False):
        self.w = workload
        self.pool = _lib.KVPool(workload.pool_slots)
        self.tree = _lib.RadixTree(self.pool)
        self.device = device
        self.use_plan = use_plan
        self.num_splits = num_splits
        self.on_extend = on_extend
        self.on_decode = on_decode
        self.min_members = min_members
        self.split_keys = split_keys
        self.host_slots = host_slots   # decode reads new slots from pinned host memory
        self.noalloc = noalloc         # decode through the entry point without a workspace
        self._ws = None
        self.content = np.full(workload.pool_slots, -1, np.int64)   # harness bookkeeping
        self.row_stride = max(len(r.tokens) + len(r.out_tokens) for r in workload.requests)
        self.dirty = []
        self.dev = None
        if device is not None:
            max_batch = max(min(p.batch_limit, len(p.rids)) for p in workload.phases)
            stride = max(len(r.tokens) + len(r.out_tokens) for r in workload.requests)
            self.dev = DeviceState(workload, device, max_batch, stride)

    # ------------------------------------------------------------------ host
    def run(self) -> EpisodeLog:
        log = EpisodeLog()
        for p_idx, ph in enumerate(self.w.phases):
            self.run_phase(p_idx, ph, list(ph.rids), log)
        log.free_list = self.pool.free_list()
        log.stats = self.tree.stats()
        return log

    def run_phase(self, p_idx, ph, rids, log: EpisodeLog) -> None:
        """Serve the requests `rids` of phase `ph` in rounds (order, admit up to the batch
        limit, extend, decode, finish), appending each round to `log`."""
        w = self.w
        waiting = list(rids)
        while waiting:
            order = self.tree.sched_order([w.requests[r].tokens for r in waiting], ph.policy)
            waiting = [waiting[i] for i in order]
            cand = waiting[:ph.batch_limit]
            k, rows, pl, nodes = self.tree.admit_batch([w.requests[r].tokens for r in cand],
                                                       ph.batch_limit, self.row_stride)
            adm: List[Admission] = [
                Admission(rid, int(pl[i]), len(w.requests[rid].tokens),
                          rows[i, :len(w.requests[rid].tokens)].copy(), int(nodes[i]))
                for i, rid in enumerate(cand[:k])]
            if not adm:
                raise RuntimeError(f"request {waiting[0]} cannot be admitted into an idle pool")
            taken = {a.rid for a in adm}
            waiting = [r for r in waiting if r not in taken]
            rnd = RoundLog(p_idx, adm, np.zeros((ph.n_decode, len(adm)), np.int32),
                           np.zeros(len(adm), np.int64))
            self._round(rnd, ph)
            log.rounds.append(rnd)

    def _round(self, rnd: RoundLog, ph):
        w = self.w
        B = len(rnd.admissions)
        for a in rnd.admissions:
            r = w.requests[a.rid]
            self.content[a.row[a.prefix_len:]] = r.kv_ids[a.prefix_len:]
        device = self.dev is not None and ph.extend != "host"
        if device:
            self._device_extend(rnd, ph)
        elif self.dev is not None:
            self.dirty.extend(a.row[a.prefix_len:] for a in rnd.admissions)
        if ph.n_decode:
            if self.use_plan and B > 1:
                rnd.plan = build_decode_plan(self.tree, [a.node for a in rnd.admissions],
                                             self.min_members, self.split_keys)
            for s in range(ph.n_decode):
                slots = self.tree.alloc(B)
                rnd.decode_slots[s] = slots
                for b, a in enumerate(rnd.admissions):
                    self.content[slots[b]] = w.requests[a.rid].out_kv_ids[s]
                if device:
                    self._device_decode(rnd, ph, s, slots)
                elif self.dev is not None:
                    self.dirty.append(slots.copy())
        seqs, rows = [], np.zeros((B, self.row_stride), np.int32)
        for b, a in enumerate(rnd.admissions):
            r = w.requests[a.rid]
            seqs.append(np.concatenate([r.tokens, r.out_tokens[:ph.n_decode]]))
            rows[b, :a.prompt_len] = a.row
            rows[b, a.prompt_len:a.prompt_len + ph.n_decode] = rnd.decode_slots[:, b]
        rnd.already_cached[:] = self.tree.finish_batch(seqs, rows, [a.prefix_len for a in rnd.admissions],
                                                       [a.node for a in rnd.admissions])

    # ---------------------------------------------------------------- device
    def _flush_dirty(self):
        """Store the K/V of slots filled during host-only phases (what those phases'
        extends would have written)."""
        d = self.dev
        if not self.dirty:
            return
        slots = np.unique(np.concatenate(self.dirty))
        slots = slots[self.content[slots] >= 0]
        self.dirty = []
        if not len(slots):
            return
        rows = d.rows_of(self.w, self.content[slots])
        _lib.kv_store(d.shape, d.kv, d.k_tab[rows], None if d.v_tab is None else d.v_tab[rows],
                      None if d.sc_tab is None else d.sc_tab[rows], d.i32(slots))

    def _device_extend(self, rnd: RoundLog, ph):
        torch = self.dev.torch
        d, w = self.dev, self.w
        self._flush_dirty()
        adm = rnd.admissions
        B = len(adm)
        host_rtt = np.zeros((B, d.rtt_stride), np.int32)
        pl = np.array([a.prefix_len for a in adm], np.int32)
        el = np.array([a.prompt_len - a.prefix_len for a in adm], np.int32)
        cu = np.zeros(B + 1, np.int32)
        cu[1:] = np.cumsum(el)
        for b, a in enumerate(adm):
            host_rtt[b, :a.prompt_len] = a.row
        d.rtt[:B].copy_(torch.from_numpy(host_rtt))
        T = int(cu[-1])
        if T == 0:
            if self.on_extend:
                self.on_extend(rnd, None, None, cu)
            return
        ids = np.concatenate([w.requests[a.rid].kv_ids[a.prefix_len:] for a in adm])
        rows = d.rows_of(w, ids)
        k_new = d.k_tab[rows]
        v_new = None if d.v_tab is None else d.v_tab[rows]
        sc_new = None if d.sc_tab is None else d.sc_tab[rows]
        if ph.extend == "store":
            slots = np.concatenate([a.row[a.prefix_len:] for a in adm])
            _lib.kv_store(d.shape, d.kv, k_new, v_new, sc_new, d.i32(slots))
            return
        qi = np.concatenate([w.q_index(a.rid, np.arange(a.prefix_len, a.prompt_len)) for a in adm])
        q = d.q_tab[torch.from_numpy(qi).to(d.device)]
        s = w.shape
        out = torch.empty((T, s.num_q_heads, s.head_dim_v), dtype=d.q_dtype, device=d.device)
        lse = torch.empty((T, s.num_q_heads), dtype=torch.float32, device=d.device)
        _lib.attn_extend(d.shape, d.kv, q, k_new, v_new, sc_new, d.rtt, None, d.i32(pl),
                         d.i32(el), d.i32(cu), B, T, int(el.max()), out, lse)
        if self.on_extend:
            self.on_extend(rnd, out, lse, cu)

    def _device_decode(self, rnd: RoundLog, ph, step, slots):
        torch = self.dev.torch
        d, w = self.dev, self.w
        if step == 0:
            self._flush_dirty()
            if ph.extend == "host":
                B = len(rnd.admissions)
                host_rtt = np.zeros((B, d.rtt_stride), np.int32)
                for b, a in enumerate(rnd.admissions):
                    host_rtt[b, :a.prompt_len] = a.row
                d.rtt[:B].copy_(torch.from_numpy(host_rtt))
            self._plan_dev = _lib.device_plan(rnd.plan, d.device) if rnd.plan is not None else (None, [])
        adm = rnd.admissions
        B = len(adm)
        s = w.shape
        seq = np.array([a.prompt_len + step + 1 for a in adm], np.int32)
        qi = np.array([w.q_index(a.rid, np.array([a.prompt_len + step]))[0] for a in adm])
        q = d.q_tab[torch.from_numpy(qi).to(d.device)]
        ids = np.array([w.requests[a.rid].out_kv_ids[step] for a in adm], np.int64)
        rows = d.rows_of(w, ids)
        k_new = d.k_tab[rows]
        v_new = None if d.v_tab is None else d.v_tab[rows]
        sc_new = None if d.sc_tab is None else d.sc_tab[rows]
        plan, _keep = self._plan_dev
        splits = self.num_splits or 0
        if not self.noalloc:
            ws_bytes = _lib.decode_workspace_size(d.shape, B, int(seq.max()), plan, splits)
            # one workspace for every call (grown when a round needs more): the bf16 merge
            # counters are zeroed once, at allocation, and every call leaves them zero
            if self._ws is None or self._ws.numel() * 4 < ws_bytes:
                self._ws = torch.zeros(max(ws_bytes // 4, 1), dtype=torch.float32, device=d.device)
        ws = self._ws
        out = torch.empty((B, s.num_q_heads, s.head_dim_v), dtype=d.q_dtype, device=d.device)
        lse = torch.empty((B, s.num_q_heads), dtype=torch.float32, device=d.device)
        if self.host_slots:
            new_slots = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).pin_memory()
        else:
            new_slots = d.i32(slots)
        if self.noalloc:
            _lib.attn_decode_noalloc(d.shape, d.kv, q, k_new, v_new, sc_new, new_slots, d.rtt,
                                     None, d.i32(seq), B, int(seq.max()), plan, splits, out, lse)
        else:
            _lib.attn_decode(d.shape, d.kv, q, k_new, v_new, sc_new, new_slots, d.rtt, None,
                             d.i32(seq), B, int(seq.max()), plan, splits, out, lse, ws)
        if self.host_slots:
            torch.cuda.current_stream().synchronize()   # the pinned slots are read by the kernel
        if self.on_decode:
            self.on_decode(rnd, step, out, lse)
