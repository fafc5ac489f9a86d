"""ctypes binding of libradix_attn.so (argument marshalling only).

Every step of the path runs in the native library: the host tree, pool and
scheduler in C++, the attention in HIP kernels. This module only converts
numpy arrays / torch tensors to pointers and status codes to exceptions. It
raises if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import sys
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RADIX_ATTN_LIB may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("RADIX_ATTN_LIB") or os.path.join(_HERE, "libradix_attn.so")

OK, E_INVAL, E_NOMEM, E_HIP, E_UNSUPPORTED = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_vp = C.c_void_p


class RadixError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"radix status {status}: {msg}")
        self.status = status


class NoMemory(RadixError):
    pass


class TreeStats(C.Structure):
    _fields_ = [("cached_tokens", C.c_int64), ("evictable_tokens", C.c_int64),
                ("num_nodes", C.c_int64), ("evicted_tokens_total", C.c_int64), ("tick", C.c_int64),
                ("pinned_tokens", C.c_int64)]


class AttnShape(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim_qk", C.c_int32),
                ("head_dim_v", C.c_int32), ("q_dtype", C.c_int32), ("kv_dtype", C.c_int32),
                ("v_is_k_prefix", C.c_int32), ("sm_scale", C.c_float)]


class KVBuffers(C.Structure):
    _fields_ = [("k_pool", _vp), ("v_pool", _vp), ("kv_scale", _vp), ("num_slots", C.c_int64)]


class DecodePlan(C.Structure):
    _fields_ = [("num_segments", C.c_int32), ("num_member_entries", C.c_int32),
                ("seg_row", _vp), ("seg_start", _vp), ("seg_end", _vp), ("seg_member_off", _vp),
                ("seg_members", _vp), ("seg_member_slot", _vp), ("seg_split_off", _vp),
                ("seg_member_part", _vp), ("seg_items", _vp), ("req_num_shared", _vp),
                ("req_num_parts", _vp),
                ("req_private_start", _vp), ("req_order", _vp), ("max_members", C.c_int32),
                ("max_shared", C.c_int32), ("max_seg_len", C.c_int32),
                ("min_private_start", C.c_int32), ("num_seg_items", C.c_int32),
                ("max_parts", C.c_int32), ("max_seg_splits", C.c_int32)]

# array fields of a plan, in DecodePlan order
_PLAN_ARRAYS = ("seg_row", "seg_start", "seg_end", "seg_member_off", "seg_members",
                "seg_member_slot", "seg_split_off", "seg_member_part", "seg_items",
                "req_num_shared", "req_num_parts", "req_private_start", "req_order")


_SIGS = {
    "radix_last_error": (C.c_char_p, []),
    "radix_version": (C.c_char_p, []),
    "radix_kv_pool_create": (C.c_int, [C.c_int64, C.POINTER(_vp)]),
    "radix_kv_pool_destroy": (None, [_vp]),
    "radix_kv_pool_alloc": (C.c_int, [_vp, C.c_int64, _i32p]),
    "radix_kv_pool_free": (C.c_int, [_vp, _i32p, C.c_int64]),
    "radix_kv_pool_num_free": (C.c_int64, [_vp]),
    "radix_kv_pool_num_slots": (C.c_int64, [_vp]),
    "radix_kv_pool_free_list": (C.c_int, [_vp, _i32p, C.c_int64, _i64p]),
    "radix_tree_create": (C.c_int, [_vp, C.POINTER(_vp)]),
    "radix_tree_destroy": (None, [_vp]),
    "radix_tree_peek": (C.c_int, [_vp, _i32p, C.c_int64, _i64p]),
    "radix_tree_match": (C.c_int, [_vp, _i32p, C.c_int64, _i64p, _i32p, _i64p]),
    "radix_tree_lock": (C.c_int, [_vp, C.c_int64]),
    "radix_tree_unlock": (C.c_int, [_vp, C.c_int64]),
    "radix_tree_alloc": (C.c_int, [_vp, C.c_int64, _i32p]),
    "radix_tree_insert": (C.c_int, [_vp, _i32p, _i32p, C.c_int64, _i64p]),
    "radix_tree_evict": (C.c_int, [_vp, C.c_int64, _i64p]),
    "radix_tree_stats_get": (C.c_int, [_vp, C.POINTER(TreeStats)]),
    "radix_sched_order": (C.c_int, [_vp, C.POINTER(_i32p), _i64p, C.c_int64, C.c_int32, _i64p]),
    "radix_req_admit": (C.c_int, [_vp, _i32p, C.c_int64, _i32p, _i64p, _i64p]),
    "radix_route": (C.c_int, [C.POINTER(_vp), C.c_int32, _i64p, _i32p, C.c_int64, C.c_int32,
                              C.c_int64, C.c_double, _i64p, _i32p, _i64p]),
    "radix_req_finish": (C.c_int, [_vp, _i32p, _i32p, C.c_int64, C.c_int64, C.c_int64, _i64p]),
    "radix_req_admit_batch": (C.c_int, [_vp, _i32p, _i64p, C.c_int64, C.c_int64, _i32p, C.c_int64,
                                        _i64p, _i64p, _i64p]),
    "radix_req_finish_batch": (C.c_int, [_vp, _i32p, _i64p, _i32p, C.c_int64, _i64p, _i64p,
                                         C.c_int64, _i64p]),
    "radix_probe_read": (C.c_int, [_vp, C.c_int64, _vp, _vp]),
    "radix_fence_create": (C.c_int, [C.POINTER(_vp)]),
    "radix_fence_record": (C.c_int, [_vp, _vp]),
    "radix_fence_wait": (C.c_int, [_vp]),
    "radix_fence_destroy": (None, [_vp]),
    "radix_profile_enable": (C.c_int, [C.c_int32]),
    "radix_profile_read": (C.c_int, [_i32p, C.POINTER(C.c_float), C.c_int32, _i32p]),
    "radix_kernel_name": (C.c_char_p, [C.c_int32]),
    "radix_tree_decode_plan": (C.c_int, [_vp, _i64p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32] + [_i32p] * 20),
    "radix_attn_supported": (C.c_int, [C.POINTER(AttnShape), C.c_int]),
    "radix_kv_store": (C.c_int, [C.POINTER(AttnShape), C.POINTER(KVBuffers), _vp, _vp, _vp, _vp,
                                 C.c_int64, _vp]),
    "radix_attn_decode_workspace_size": (C.c_int, [C.POINTER(AttnShape), C.c_int32, C.c_int32,
                                                   C.POINTER(DecodePlan), C.c_int32,
                                                   C.POINTER(C.c_size_t)]),
    "radix_attn_extend": (C.c_int, [C.POINTER(AttnShape), C.POINTER(KVBuffers), _vp, _vp, _vp, _vp,
                                    _vp, C.c_int32, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                    C.c_int32, _vp, _vp, _vp]),
    "radix_attn_decode": (C.c_int, [C.POINTER(AttnShape), C.POINTER(KVBuffers), _vp, _vp, _vp, _vp,
                                    _vp, _vp, C.c_int32, _vp, _vp, C.c_int32, C.c_int32,
                                    C.POINTER(DecodePlan), C.c_int32, _vp, _vp, _vp, C.c_size_t,
                                    _vp]),
    "radix_attn_decode_noalloc": (C.c_int, [C.POINTER(AttnShape), C.POINTER(KVBuffers), _vp, _vp,
                                            _vp, _vp, _vp, _vp, C.c_int32, _vp, _vp, C.c_int32,
                                            C.c_int32, C.POINTER(DecodePlan), C.c_int32, _vp, _vp,
                                            _vp]),
    "radix_attn_decode_noalloc_max_bytes": (C.c_size_t, []),
}

_LIB = None


def load():
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m prefix_shared_kv_radix_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def exported_symbols():
    return list(_SIGS)


def _check(status):
    if status != OK:
        msg = load().radix_last_error().decode(errors="replace")
        if status == E_NOMEM:
            raise NoMemory(status, msg)
        raise RadixError(status, msg)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


# ---------------------------------------------------------------------- host
class KVPool:
    """Slot pool (host). Owns the native object."""

    def __init__(self, num_slots: int):
        lib = load()
        h = _vp()
        _check(lib.radix_kv_pool_create(int(num_slots), C.byref(h)))
        self.h = h

    def close(self):
        if self.h and not sys.is_finalizing():
            load().radix_kv_pool_destroy(self.h)
        self.h = None

    __del__ = close

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(int(n), np.int32)
        _check(load().radix_kv_pool_alloc(self.h, int(n), out.ctypes.data_as(_i32p)))
        return out

    def free(self, slots) -> None:
        a, p = _i32(slots)
        _check(load().radix_kv_pool_free(self.h, p, len(a)))

    def num_free(self) -> int:
        return int(load().radix_kv_pool_num_free(self.h))

    def free_list(self) -> np.ndarray:
        n = C.c_int64()
        cap = self.num_free()
        out = np.empty(max(cap, 1), np.int32)
        _check(load().radix_kv_pool_free_list(self.h, out.ctypes.data_as(_i32p), cap, C.byref(n)))
        return out[:n.value].copy()


class RadixTree:
    """Radix tree over token ids (host). Keeps its pool alive."""

    def __init__(self, pool: KVPool):
        lib = load()
        h = _vp()
        _check(lib.radix_tree_create(pool.h, C.byref(h)))
        self.h = h
        self.pool = pool

    def close(self):
        if self.h and not sys.is_finalizing():
            load().radix_tree_destroy(self.h)
        self.h = None

    __del__ = close

    def peek(self, tokens) -> int:
        a, p = _i32(tokens)
        m = C.c_int64()
        _check(load().radix_tree_peek(self.h, p, len(a), C.byref(m)))
        return m.value

    def match(self, tokens):
        a, p = _i32(tokens)
        m, node = C.c_int64(), C.c_int64()
        out = np.empty(max(len(a), 1), np.int32)
        _check(load().radix_tree_match(self.h, p, len(a), C.byref(m), out.ctypes.data_as(_i32p),
                                       C.byref(node)))
        return m.value, out[:m.value].copy(), node.value

    def lock(self, node):
        _check(load().radix_tree_lock(self.h, int(node)))

    def unlock(self, node):
        _check(load().radix_tree_unlock(self.h, int(node)))

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(max(int(n), 1), np.int32)
        _check(load().radix_tree_alloc(self.h, int(n), out.ctypes.data_as(_i32p)))
        return out[:int(n)]

    def insert(self, tokens, slots) -> int:
        a, pa = _i32(tokens)
        b, pb = _i32(slots)
        if len(a) != len(b):
            raise ValueError("tokens and slots differ in length")
        c = C.c_int64()
        _check(load().radix_tree_insert(self.h, pa, pb, len(a), C.byref(c)))
        return c.value

    def evict(self, n: int) -> int:
        f = C.c_int64()
        _check(load().radix_tree_evict(self.h, int(n), C.byref(f)))
        return f.value

    def stats(self) -> TreeStats:
        s = TreeStats()
        _check(load().radix_tree_stats_get(self.h, C.byref(s)))
        return s

    def sched_order(self, prompts, policy: str):
        arrs = [np.ascontiguousarray(p, dtype=np.int32) for p in prompts]
        n = len(arrs)
        ptrs = (_i32p * max(n, 1))(*[a.ctypes.data_as(_i32p) for a in arrs])
        lens = np.array([len(a) for a in arrs], np.int64)
        out = np.empty(max(n, 1), np.int64)
        code = {"fcfs": 0, "lpf": 1}[policy]
        _check(load().radix_sched_order(self.h, ptrs, lens.ctypes.data_as(_i64p), n, code,
                                        out.ctypes.data_as(_i64p)))
        return out[:n].tolist()

    def admit(self, tokens):
        """(prefix_len, row slots, node); raises NoMemory (request stays waiting)."""
        a, p = _i32(tokens)
        row = np.empty(max(len(a), 1), np.int32)
        m, node = C.c_int64(), C.c_int64()
        st = load().radix_req_admit(self.h, p, len(a), row.ctypes.data_as(_i32p), C.byref(m),
                                    C.byref(node))
        _check(st)
        return m.value, row[:len(a)], node.value

    def finish(self, tokens, row, prefix_len, node) -> int:
        a, pa = _i32(tokens)
        b, pb = _i32(row)
        c = C.c_int64()
        _check(load().radix_req_finish(self.h, pa, pb, len(a), int(prefix_len), int(node),
                                       C.byref(c)))
        return c.value

    def admit_batch(self, prompts, max_batch: int, row_stride: int):
        """Admit prompts in order until max_batch or a request cannot get its slots.
        Returns (count, rows [count, row_stride], prefix_len [count], nodes [count])."""
        n = min(len(prompts), int(max_batch))
        prompts = prompts[:n]
        off = np.zeros(n + 1, np.int64)
        off[1:] = np.cumsum([len(p) for p in prompts])
        flat = np.ascontiguousarray(np.concatenate(prompts) if n else np.zeros(1, np.int32),
                                    dtype=np.int32)
        rows = np.zeros((max(n, 1), int(row_stride)), np.int32)
        pl = np.zeros(max(n, 1), np.int64)
        nodes = np.zeros(max(n, 1), np.int64)
        k = C.c_int64()
        _check(load().radix_req_admit_batch(self.h, flat.ctypes.data_as(_i32p),
                                            off.ctypes.data_as(_i64p), n, n,
                                            rows.ctypes.data_as(_i32p), int(row_stride),
                                            pl.ctypes.data_as(_i64p), nodes.ctypes.data_as(_i64p),
                                            C.byref(k)))
        k = k.value
        return k, rows[:k], pl[:k], nodes[:k]

    def finish_batch(self, seqs, rows, prefix_len, nodes):
        """Finish requests: seqs[i] = prompt + outputs, rows[i, :len(seqs[i])] their slots."""
        n = len(seqs)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        off = np.zeros(n + 1, np.int64)
        off[1:] = np.cumsum([len(x) for x in seqs])
        flat = np.ascontiguousarray(np.concatenate(seqs) if n else np.zeros(1, np.int32),
                                    dtype=np.int32)
        pl = np.ascontiguousarray(prefix_len, dtype=np.int64)
        nd = np.ascontiguousarray(nodes, dtype=np.int64)
        out = np.zeros(max(n, 1), np.int64)
        _check(load().radix_req_finish_batch(self.h, flat.ctypes.data_as(_i32p),
                                             off.ctypes.data_as(_i64p), rows.ctypes.data_as(_i32p),
                                             rows.shape[1] if rows.ndim == 2 else 0,
                                             pl.ctypes.data_as(_i64p), nd.ctypes.data_as(_i64p), n,
                                             out.ctypes.data_as(_i64p)))
        return out[:n]

    def decode_plan(self, nodes, min_members: int = 2, split_keys: int = 0):
        """Shared-segment plan (host arrays) for requests admitted at `nodes`; segments
        longer than split_keys keys are cut into chunks (0: one chunk per segment)."""
        nodes = np.ascontiguousarray(nodes, dtype=np.int64)
        B = len(nodes)
        cap_seg = max(2 * B, 1)
        cap_mem = max(B * 8, 1)
        cap_items = max(4 * B, 1)
        while True:
            # seg_row, seg_start, seg_end [cap_seg]; seg_member_off, seg_split_off [cap_seg+1]
            seg = [np.zeros(cap_seg + (1 if k >= 3 else 0), np.int32) for k in range(5)]
            # seg_members, seg_member_slot, seg_member_part [cap_mem]
            mem = [np.zeros(cap_mem, np.int32) for _ in range(3)]
            items = np.zeros(cap_items * 8, np.int32)   # chunk records
            # req_num_shared, req_num_parts, req_private_start, req_order [batch]
            req = [np.zeros(max(B, 1), np.int32) for _ in range(4)]
            cnt = [C.c_int32() for _ in range(7)]
            p = lambda x: x.ctypes.data_as(_i32p)
            st = load().radix_tree_decode_plan(
                self.h, nodes.ctypes.data_as(_i64p), B, int(min_members), int(split_keys),
                cap_seg, cap_mem, cap_items, p(seg[0]), p(seg[1]), p(seg[2]), p(seg[3]),
                p(mem[0]), p(mem[1]), p(seg[4]), p(mem[2]), p(items), p(req[0]), p(req[1]),
                p(req[2]), p(req[3]), *[C.byref(c) for c in cnt])
            ns, nm, ni = cnt[0].value, cnt[1].value, cnt[4].value
            if st == E_INVAL and (ns > cap_seg or nm > cap_mem or ni > cap_items):
                cap_seg, cap_mem, cap_items = max(cap_seg, ns), max(cap_mem, nm), max(cap_items, ni)
                continue
            _check(st)
            break
        return HostPlan(seg_row=seg[0][:ns], seg_start=seg[1][:ns], seg_end=seg[2][:ns],
                        seg_member_off=seg[3][:ns + 1] if ns else np.zeros(1, np.int32),
                        seg_members=mem[0][:nm], seg_member_slot=mem[1][:nm],
                        seg_split_off=seg[4][:ns + 1] if ns else np.zeros(1, np.int32),
                        seg_member_part=mem[2][:nm], seg_items=items[:8 * ni],
                        req_num_shared=req[0][:B], req_num_parts=req[1][:B],
                        req_private_start=req[2][:B], req_order=req[3][:B],
                        max_members=cnt[2].value, max_shared=cnt[3].value,
                        num_seg_items=cnt[4].value, max_parts=cnt[5].value,
                        max_seg_splits=cnt[6].value)


ROUTE_POLICIES = {"round_robin": 0, "cache_aware": 1, "least_load": 2}


class Router:
    """Data-parallel request routing over several trees (one per worker)."""

    def __init__(self, trees, policy: str, balance_abs: int = 32, balance_rel: float = 1.5):
        self.trees = list(trees)
        self.policy = ROUTE_POLICIES[policy]
        self.balance_abs = int(balance_abs)
        self.balance_rel = float(balance_rel)
        self.rr = C.c_int64(0)

    def route(self, tokens, loads):
        """(worker index, that worker's cached prefix length) for one request."""
        a, p = _i32(tokens)
        ld = np.ascontiguousarray(loads, dtype=np.int64)
        hs = (_vp * len(self.trees))(*[t.h for t in self.trees])
        wk, m = C.c_int32(), C.c_int64()
        _check(load().radix_route(hs, len(self.trees), ld.ctypes.data_as(_i64p), p, len(a),
                                  self.policy, self.balance_abs, self.balance_rel,
                                  C.byref(self.rr), C.byref(wk), C.byref(m)))
        return wk.value, m.value


@dataclass
class HostPlan:
    seg_row: np.ndarray
    seg_start: np.ndarray
    seg_end: np.ndarray
    seg_member_off: np.ndarray
    seg_members: np.ndarray
    seg_member_slot: np.ndarray
    seg_split_off: np.ndarray
    seg_member_part: np.ndarray
    seg_items: np.ndarray
    req_num_shared: np.ndarray
    req_num_parts: np.ndarray
    req_private_start: np.ndarray
    req_order: np.ndarray
    max_members: int
    max_shared: int
    num_seg_items: int
    max_parts: int
    max_seg_splits: int

    @property
    def num_segments(self):
        return len(self.seg_row)

    @property
    def min_private_start(self):
        return int(self.req_private_start.min()) if len(self.req_private_start) else 0

    @property
    def max_seg_len(self):
        return int((self.seg_end - self.seg_start).max()) if len(self.seg_row) else 0


# ---------------------------------------------------------------------- device
def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def make_shape(num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, q_dtype, kv_dtype,
               v_is_k_prefix, sm_scale) -> AttnShape:
    return AttnShape(num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, DTYPE_CODES[q_dtype],
                     DTYPE_CODES[kv_dtype], int(bool(v_is_k_prefix)), float(sm_scale))


def make_kv(k_pool, v_pool, kv_scale) -> KVBuffers:
    return KVBuffers(_ptr(k_pool), _ptr(v_pool), _ptr(kv_scale), int(k_pool.shape[0]))


def attn_supported(shape: AttnShape, is_decode: bool) -> bool:
    return load().radix_attn_supported(C.byref(shape), int(is_decode)) == OK


def kv_store(shape, kv, k_new, v_new, scale_new, slots, stream=None):
    _check(load().radix_kv_store(C.byref(shape), C.byref(kv), _ptr(k_new), _ptr(v_new),
                                 _ptr(scale_new), _ptr(slots), int(slots.numel()), _stream(stream)))


def host_plan_struct(plan):
    """DecodePlan carrying only the host scalars of a HostPlan (for workspace queries)."""
    if plan is None or plan.num_segments == 0:
        return None
    return DecodePlan(plan.num_segments, len(plan.seg_members), *([None] * len(_PLAN_ARRAYS)),
                      plan.max_members, plan.max_shared, plan.max_seg_len,
                      plan.min_private_start, plan.num_seg_items, plan.max_parts,
                      plan.max_seg_splits)


def decode_workspace_size(shape, batch, max_seq_len, plan, num_splits) -> int:
    """plan: a HostPlan, a DecodePlan or None."""
    if isinstance(plan, HostPlan):
        plan = host_plan_struct(plan)
    n = C.c_size_t()
    _check(load().radix_attn_decode_workspace_size(C.byref(shape), int(batch), int(max_seq_len),
                                                   None if plan is None else C.byref(plan),
                                                   int(num_splits), C.byref(n)))
    return n.value


def attn_extend(shape, kv, q, k_new, v_new, scale_new, req_to_token, req_rows, prefix_lens,
                extend_lens, cu_extend, batch, total_extend, max_extend, out, lse_out=None,
                stream=None):
    _check(load().radix_attn_extend(
        C.byref(shape), C.byref(kv), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale_new),
        _ptr(req_to_token), int(req_to_token.shape[1]), _ptr(req_rows), _ptr(prefix_lens),
        _ptr(extend_lens), _ptr(cu_extend), int(batch), int(total_extend), int(max_extend),
        _ptr(out), _ptr(lse_out), _stream(stream)))


def device_plan(plan: HostPlan, device):
    """Upload a HostPlan; returns (DecodePlan struct, tensors kept alive by the caller)."""
    import torch
    if plan is None or plan.num_segments == 0:
        return None, []
    # all arrays in one pinned buffer and one asynchronous copy: a copy from pageable
    # memory would make the host wait for everything already queued on the stream
    arrays = [np.ascontiguousarray(getattr(plan, f), dtype=np.int32) for f in _PLAN_ARRAYS]
    offs = np.concatenate([[0], np.cumsum([len(x) for x in arrays])])
    host = torch.empty(max(int(offs[-1]), 1), dtype=torch.int32, pin_memory=True)
    hv = host.numpy()
    for x, o in zip(arrays, offs[:-1]):
        hv[o:o + len(x)] = x
    dev = torch.empty_like(host, device=device)
    dev.copy_(host, non_blocking=True)
    base = dev.data_ptr()
    dp = DecodePlan(plan.num_segments, len(plan.seg_members),
                    *[_vp(base + 4 * int(o)) for o in offs[:-1]],
                    plan.max_members, plan.max_shared, plan.max_seg_len, plan.min_private_start,
                    plan.num_seg_items, plan.max_parts, plan.max_seg_splits)
    return dp, [dev, host]


def attn_decode(shape, kv, q, k_new, v_new, scale_new, new_slots, req_to_token, req_rows, seq_lens,
                batch, max_seq_len, plan, num_splits, out, lse_out, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().radix_attn_decode(
        C.byref(shape), C.byref(kv), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale_new),
        _ptr(new_slots), _ptr(req_to_token), int(req_to_token.shape[1]), _ptr(req_rows),
        _ptr(seq_lens), int(batch), int(max_seq_len), None if plan is None else C.byref(plan),
        int(num_splits), _ptr(out), _ptr(lse_out), _ptr(workspace), ws_bytes, _stream(stream)))


def probe_read(buf, sink, stream=None):
    """Read the device tensor `buf` once (radix_probe_read); `sink`: >= 8192 int32 on the
    device."""
    if buf.numel() * buf.element_size() % 16 or sink.numel() < 8192:
        raise ValueError("probe_read: buffer bytes must be a multiple of 16, sink >= 8192 words")
    _check(load().radix_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                   _stream(stream)))


def attn_decode_noalloc(shape, kv, q, k_new, v_new, scale_new, new_slots, req_to_token, req_rows,
                        seq_lens, batch, max_seq_len, plan, num_splits, out, lse_out, stream=None):
    """radix_attn_decode without a workspace (the library's built-in scratch array)."""
    _check(load().radix_attn_decode_noalloc(
        C.byref(shape), C.byref(kv), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale_new),
        _ptr(new_slots), _ptr(req_to_token), int(req_to_token.shape[1]), _ptr(req_rows),
        _ptr(seq_lens), int(batch), int(max_seq_len), None if plan is None else C.byref(plan),
        int(num_splits), _ptr(out), _ptr(lse_out), _stream(stream)))


def decode_noalloc_max_bytes() -> int:
    return int(load().radix_attn_decode_noalloc_max_bytes())


class Fence:
    """A point in a stream the host can wait for (device-scope release only)."""

    def __init__(self):
        h = _vp()
        _check(load().radix_fence_create(C.byref(h)))
        self.h = h

    def record(self, stream=None):
        _check(load().radix_fence_record(self.h, _stream(stream)))

    def wait(self):
        _check(load().radix_fence_wait(self.h))

    def close(self):
        if self.h and not sys.is_finalizing():
            load().radix_fence_destroy(self.h)
        self.h = None

    __del__ = close


# ---------------------------------------------------------------------- timing
def profile_enable(capacity: int) -> None:
    _check(load().radix_profile_enable(int(capacity)))


def profile_read(cap: int = 1 << 16):
    """[(kernel name, milliseconds)] for the launches recorded since the last read."""
    ids = np.zeros(cap, np.int32)
    ms = np.zeros(cap, np.float32)
    n = C.c_int32()
    _check(load().radix_profile_read(ids.ctypes.data_as(_i32p),
                                     ms.ctypes.data_as(C.POINTER(C.c_float)), cap, C.byref(n)))
    lib = load()
    return [(lib.radix_kernel_name(int(i)).decode(), float(t)) for i, t in zip(ids[:n.value], ms[:n.value])]
