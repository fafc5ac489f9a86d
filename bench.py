"""Throughput of prefix-shared KV attention over a radix-tree slot pool on one MI355X.

One step = one whole episode of the workload: for every round, order and admit
the requests through the native radix tree (match, pin, allocate with LRU
eviction), extend them (store new K/V + attention against the cached prefix),
run every decode step (one new slot per request from the tree, store, decode
attention over shared segments + private tails), and finish them (insert,
free duplicates, unpin). Query/K/V inputs are staged in HBM before the timed
region; slot lists are produced inside it by the host tree and copied over.

The attention runs for `--layers` layers (default 4), each with its own K/V pool and
the same slot lists, as in a model: one layer's keys (about 210 MB in the few-shot
decode step) are then not still in the 256 MB last-level cache when that layer's next
step reads them. With --layers 1 consecutive steps re-read one pool and part of it
comes from that cache. All figures are per layer.

Prints one JSON line. `value` = decode tokens generated per second of episode
time per layer (whole job); the breakdown, per-kernel event timings (taken over a second,
identical run of the same steps, since an event pair around every launch slows the
step), the roofline of the dominant kernel and the CPU oracle's rate on a bounded
sample are included.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", default="4",
                   help="4 (default: agent branching, the largest single-GPU workload), "
                        "1, 2, 2fp8, 3A, 3B, 4fp8, 5bf16, 5fp8")
    p.add_argument("--no-plan", action="store_true", help="decode without shared segments")
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--split-keys", type=int, default=None,
                   help="key chunk length of long shared segments (default: chosen per round)")
    p.add_argument("--min-members", type=int, default=2,
                   help="members a shared segment needs to be read once for all of them")
    p.add_argument("--layers", type=int, default=4,
                   help="attention layers per step, each with its own K/V pool (same contents): "
                        "together they exceed the 256 MB last-level cache, as a model's layers do")
    p.add_argument("--schedule", choices=["overlap", "sync", "free"], default="overlap",
                   help="overlap: the host prepares decode step s+1 while earlier steps run, "
                        "waiting only for step s+1-ahead; sync: it waits for each step before "
                        "the next; free: it never waits inside a round")
    p.add_argument("--ahead", type=int, default=1,
                   help="overlap: decode steps the host may run ahead of the GPU")
    p.add_argument("--no-kernel-timing", action="store_true",
                   help="skip the second, kernel-timed pass (for external profilers)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return p.parse_args()


def workload_of(name):
    from workloads import config
    table = {"1": (1, ""), "2": (2, ""), "2fp8": (2, "fp8"), "3A": (3, "A"), "3B": (3, "B"),
             "4": (4, ""), "4fp8": (4, "fp8"), "5bf16": (5, "bf16"), "5fp8": (5, "fp8")}
    n, v = table[name]
    return config(n, v)


class Episode:
    """Pre-staged device inputs for every round of a workload, and one timed pass."""

    def __init__(self, w, use_plan, splits, layers=1, schedule="overlap", ahead=1,
                 min_members=2, split_keys=None):
        import torch
        from prefix_shared_kv_radix_amd import _lib
        from prefix_shared_kv_radix_amd.runner import DeviceState, Engine, build_decode_plan
        self.torch, self._lib, self.build_plan = torch, _lib, build_decode_plan
        self.w, self.use_plan, self.splits = w, use_plan, splits
        self.min_members = min_members
        self.split_keys = split_keys
        # "overlap": the host prepares decode step s+1 (slot allocation, pinned slot rows,
        # launches) while step s runs, and waits only for step s-1 (whose outputs a server
        # would read); "sync": the host waits for every step before preparing the next
        self.schedule = schedule
        self.ahead = max(1, int(ahead))
        self.step_evt = [_lib.Fence() for _ in range(self.ahead + 1)]
        # host-only pass: the rounds (and their plans) are deterministic
        dry = Engine(w, min_members=min_members, split_keys=split_keys).run()
        self.rounds = dry.rounds
        dev = "cuda"
        max_batch = max(len(r.admissions) for r in dry.rounds)
        self.stride = max(len(r.tokens) + len(r.out_tokens) for r in w.requests)
        self.d = DeviceState(w, dev, max_batch, self.stride)
        d, s = self.d, w.shape
        # one K/V pool per layer; layers past the first get copies of the first pool's
        # initial contents, then every layer's extend and decode store their own rows
        self.layers = layers
        self.pools = [(d.k_pool, d.v_pool, d.kv_scale)] + [
            tuple(None if t is None else t.clone() for t in (d.k_pool, d.v_pool, d.kv_scale))
            for _ in range(layers - 1)]
        self.kvs = [_lib.make_kv(*p) for p in self.pools]
        self.staged = []
        self.max_ws = 0
        for r_idx, rnd in enumerate(dry.rounds):
            ph = w.phases[rnd.phase]
            adm = rnd.admissions
            B = len(adm)
            st = {"B": B, "ph": ph, "rids": [a.rid for a in adm],
                  "prompts": [w.requests[a.rid].tokens for a in adm],
                  "seqs": [np.concatenate([w.requests[a.rid].tokens,
                                           w.requests[a.rid].out_tokens[:ph.n_decode]]) for a in adm],
                  "prompt_len": np.array([a.prompt_len for a in adm], np.int32),
                  "prefix_len": np.array([a.prefix_len for a in adm], np.int64)}
            el = st["prompt_len"] - st["prefix_len"].astype(np.int32)
            cu = np.zeros(B + 1, np.int32)
            cu[1:] = np.cumsum(el)
            st.update(el=el, cu=cu, T=int(cu[-1]), max_e=int(el.max()) if B else 0,
                      pl_dev=d.i32(st["prefix_len"]), el_dev=d.i32(el), cu_dev=d.i32(cu))
            if ph.extend != "host" and st["T"]:
                ids = np.concatenate([w.requests[a.rid].kv_ids[a.prefix_len:] for a in adm])
                rows = d.rows_of(w, ids)
                st["k_new"] = d.k_tab[rows]
                st["v_new"] = None if d.v_tab is None else d.v_tab[rows]
                st["sc_new"] = None if d.sc_tab is None else d.sc_tab[rows]
                st["slots_hint"] = None
                if ph.extend == "attend":
                    qi = np.concatenate([w.q_index(a.rid, np.arange(a.prefix_len, a.prompt_len))
                                         for a in adm])
                    st["q"] = d.q_tab[torch.from_numpy(qi).to(dev)]
                    st["out"] = torch.empty((st["T"], s.num_q_heads, s.head_dim_v),
                                            dtype=d.q_dtype, device=dev)
            if ph.n_decode:
                n = ph.n_decode
                qi = np.stack([w.q_index(a.rid, a.prompt_len + np.arange(n)) for a in adm], 1)
                st["dq"] = d.q_tab[torch.from_numpy(qi.reshape(-1)).to(dev)].view(
                    n, B, s.num_q_heads, s.head_dim_qk)
                ids = np.stack([w.requests[a.rid].out_kv_ids[:n] for a in adm], 1)
                rows = d.rows_of(w, ids.reshape(-1))
                st["dk"] = d.k_tab[rows].view(n, B, *d.k_tab.shape[1:])
                st["dv"] = None if d.v_tab is None else d.v_tab[rows].view(n, B, *d.v_tab.shape[1:])
                st["dsc"] = None if d.sc_tab is None else d.sc_tab[rows].view(n, B)
                seq = st["prompt_len"][None, :] + 1 + np.arange(n)[:, None]
                st["seq_dev"] = d.i32(seq)
                st["seq_host"] = seq
                st["seq_max"] = [int(x) for x in seq.max(axis=1)]
                st["dout"] = torch.empty((B, s.num_q_heads, s.head_dim_v), dtype=d.q_dtype, device=dev)
                st["slot_pin"] = torch.empty((2, n, B), dtype=torch.int32, pin_memory=True)
                st["slot_dev"] = torch.empty((n, B), dtype=torch.int32, device=dev)
                plan = rnd.plan if use_plan else None
                self.max_ws = max(self.max_ws, _lib.decode_workspace_size(
                    d.shape, B, int(seq.max()), plan, splits))
            self.staged.append(st)
        # zeroed once: the bf16 decode's merge counters must start at zero (calls leave them so)
        self.ws = torch.zeros(max(self.max_ws // 4, 1), dtype=torch.float32, device=dev)
        self.rtt_pin = torch.empty((2, max_batch, self.stride), dtype=torch.int32, pin_memory=True)
        self.parity = 0
        self.done_evt = [None, None]
        self.marks = []

    def run(self, mark=False):
        """One episode; returns nothing (all work is enqueued on the current stream)."""
        torch, _lib, d, w = self.torch, self._lib, self.d, self.w
        par = self.parity
        self.parity ^= 1
        if self.done_evt[par] is not None:
            self.done_evt[par].synchronize()       # pinned staging of two episodes ago is free
        pool = _lib.KVPool(w.pool_slots)
        tree = _lib.RadixTree(pool)
        rtt_pin = self.rtt_pin[par]
        marks = []
        for st in self.staged:
            ph, B = st["ph"], st["B"]
            k, rows, pl, nodes = tree.admit_batch(st["prompts"], B, self.stride)
            if k != B or not np.array_equal(pl, st["prefix_len"]):
                raise RuntimeError("episode diverged from its dry run")
            plan_dev, keep = (None, [])
            if ph.n_decode and self.use_plan and B > 1:
                plan_dev, keep = _lib.device_plan(
                    self.build_plan(tree, nodes, self.min_members, self.split_keys), d.device)
            if ph.extend != "host":
                rtt_pin[:B].copy_(torch.from_numpy(rows))
                d.rtt[:B].copy_(rtt_pin[:B], non_blocking=True)
            if mark:
                marks.append(("extend_start", torch.cuda.Event(enable_timing=True)))
                marks[-1][1].record()
            if ph.extend != "host" and st["T"]:
                if ph.extend == "attend":
                    for kv in self.kvs:
                        _lib.attn_extend(d.shape, kv, st["q"], st["k_new"], st["v_new"], st["sc_new"],
                                         d.rtt, None, st["pl_dev"], st["el_dev"], st["cu_dev"], B,
                                         st["T"], st["max_e"], st["out"], None)
                else:
                    slots = d.i32(np.concatenate([rows[b, st["prefix_len"][b]:st["prompt_len"][b]]
                                                  for b in range(B)]))
                    for kv in self.kvs:
                        _lib.kv_store(d.shape, kv, st["k_new"], st["v_new"], st["sc_new"], slots)
            if mark:
                marks.append(("decode_start", torch.cuda.Event(enable_timing=True)))
                marks[-1][1].record()
            n = ph.n_decode
            if n:
                pin = st["slot_pin"][par]
                pin_np = pin.numpy()              # the pinned rows, written in place
                stream = torch.cuda.current_stream()
                cols = st["prompt_len"]
                ar = np.arange(B)
                for s in range(n):
                    slots = tree.alloc(B)
                    rows[ar, cols + s] = slots
                    pin_np[s] = slots
                    # GQA decode reads the new slots from pinned host memory (no copy launch);
                    # the MLA path stores the new rows in a separate launch first, from device memory
                    slot_arg = pin[s]
                    if w.shape.v_is_k_prefix:
                        st["slot_dev"][s].copy_(pin[s], non_blocking=True)
                        slot_arg = st["slot_dev"][s]
                    for kv in self.kvs:
                        _lib.attn_decode(d.shape, kv, st["dq"][s], st["dk"][s],
                                         None if st["dv"] is None else st["dv"][s],
                                         None if st["dsc"] is None else st["dsc"][s], slot_arg,
                                         d.rtt, None, st["seq_dev"][s], B, st["seq_max"][s],
                                         plan_dev, self.splits, st["dout"], None, self.ws, stream)
                    if self.schedule == "free":
                        continue
                    k = len(self.step_evt)
                    self.step_evt[s % k].record(stream)
                    if self.schedule == "sync":
                        self.step_evt[s % k].wait()
                    elif s >= self.ahead:
                        # step s - ahead has finished (a server reads its outputs now) while
                        # the steps after it run
                        self.step_evt[(s - self.ahead) % k].wait()
            if mark:
                marks.append(("round_end", torch.cuda.Event(enable_timing=True)))
                marks[-1][1].record()
            tree.finish_batch(st["seqs"], rows, pl, nodes)
            del keep
        evt = torch.cuda.Event()
        evt.record()
        self.done_evt[par] = evt
        if mark:
            self.marks.append(marks)
        tree.close()
        pool.close()


def algorithmic(w, ep, name):
    """Algorithmic work of one episode for a kernel family: (bytes, flops).

    Bytes count each distinct KV row a launch must read once (plus its slot index),
    queries read and final outputs written; partial results and re-reads are not
    algorithmic. Flops: 2*Hq*(Dqk+Dv) per (query, key) pair."""
    s = w.shape
    eb_kv = {"f32": 4, "bf16": 2, "fp8": 1}[s.kv_dtype]
    eb_q = {"f32": 4, "bf16": 2}[s.q_dtype]
    row_kv = s.num_kv_heads * (s.head_dim_qk + (0 if s.v_is_k_prefix else s.head_dim_v)) * eb_kv \
        + (4 if s.kv_dtype == "fp8" else 0) + 4
    q_row = s.num_q_heads * s.head_dim_qk * eb_q
    o_row = s.num_q_heads * s.head_dim_v * eb_q
    pair_flops = 2.0 * s.num_q_heads * (s.head_dim_qk + s.head_dim_v)
    byt, flop = 0.0, 0.0
    for st, rnd in zip(ep.staged, ep.rounds):
        ph, B = st["ph"], st["B"]
        if name == "extend_mfma" and ph.extend == "attend":
            for a in rnd.admissions:
                P, E = a.prefix_len, a.prompt_len - a.prefix_len
                flop += pair_flops * (E * P + E * (E + 1) / 2)
                byt += (P + E) * row_kv + E * (q_row + o_row)
        if name == "kv_store" and ph.extend != "host":
            byt += 2 * st["T"] * row_kv
        if not ph.n_decode:
            continue
        plan = rnd.plan if ep.use_plan and B > 1 else None
        seg_rows = float((plan.seg_end - plan.seg_start).sum()) if plan is not None else 0.0
        ps = plan.req_private_start if plan is not None else np.zeros(B, np.int32)
        for step in range(ph.n_decode):
            L = st["prompt_len"] + step + 1
            flop_step = pair_flops * float(L.sum())
            if name == "mla_decode":
                # distinct rows: shared prefixes once, the rest per request
                shared = seg_rows
                byt += (shared + float((L - ps).sum())) * row_kv + B * (q_row + o_row)
                flop += flop_step
            if name in ("decode_tail_valu", "decode_fused"):
                byt += float((L - ps).sum()) * row_kv + B * (q_row + o_row)
                flop += pair_flops * float((L - ps).sum())
            if name in ("segment_mfma", "decode_fused") and plan is not None:
                byt += seg_rows * row_kv
                mem = np.diff(plan.seg_member_off)
                flop += pair_flops * float(((plan.seg_end - plan.seg_start) * mem).sum())
    return byt, flop


KERNEL_DIR = os.path.join(ROOT, "prefix_shared_kv_radix_amd", "csrc", "kernels")
PROFILE_DIR = os.path.join(ROOT, "profiles")


_CODE_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src):
    """Source text with comments removed and whitespace runs collapsed (string
    literals kept): what the compiler sees, up to layout."""
    src = _CODE_TOKEN.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
    return " ".join(src.split())


def kernel_sources_digest(kernel_dir=None):
    """sha256 over the device kernel sources, comments and layout ignored: counter
    figures taken from another digest describe other code and are not reported."""
    import hashlib
    kernel_dir = kernel_dir or KERNEL_DIR
    h = hashlib.sha256()
    for f in sorted(os.listdir(kernel_dir)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(kernel_dir, f), encoding="utf-8") as fh:
                h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3
    counter summaries: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the
    kernel's dispatches), each scaled by what it reads for a plain device copy of known
    size. A summary line looks like
        traffic: kernel=K workload=W fetch_kib=F write_kib=X fetch_scale=a write_scale=b sources=D
    None when no summary matches the current kernel sources."""
    if not os.path.isdir(PROFILE_DIR):
        return None
    digest = kernel_sources_digest()
    for f in sorted(os.listdir(PROFILE_DIR)):
        if not f.endswith((".md", ".txt")):
            continue
        with open(os.path.join(PROFILE_DIR, f)) as fh:
            for line in fh:
                line = line.strip()
                if not line.startswith("traffic:"):
                    continue
                kv = dict(item.split("=", 1) for item in line[len("traffic:"):].split())
                if kv.get("kernel") == kernel and kv.get("workload") == workload \
                        and kv.get("sources") == digest:
                    return 1024.0 * (float(kv["fetch_kib"]) * float(kv["fetch_scale"])
                                     + float(kv["write_kib"]) * float(kv["write_scale"]))
    return None


def _oracle_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def _decode_queries(w, log, seconds):
    """Oracle decode queries of the workload's decode requests, step after step, for
    at most `seconds`: (queries, elapsed seconds, context length of the first)."""
    from oracle.attention import reference_outputs
    dec = [(a, len(rnd.decode_slots)) for rnd in log.rounds for a in rnd.admissions
           if len(rnd.decode_slots)]
    n = 0
    t0 = time.perf_counter()
    for step in range(max(s for _, s in dec)):
        for a, ns in dec:
            if step < ns:
                reference_outputs(w, a.rid, np.array([a.prompt_len + step]))
                n += 1
            if time.perf_counter() - t0 > seconds:
                return n, time.perf_counter() - t0, int(dec[0][0].prompt_len) + 1
    return n, time.perf_counter() - t0, int(dec[0][0].prompt_len) + 1


def cpu_baseline(w, seconds):
    """The oracle as it stands, on bounded samples of the same workload:
      - decode: fp64 decode queries of the decode requests (first step on), request
        after request, for `seconds` with the host's BLAS threads and for a quarter
        of that on one thread;
      - extend: the last extended request's new rows against its cached prefix;
      - host tree: one whole episode of matching, pinning, allocation with eviction,
        scheduling and insertion, the Python oracle against the C++ library.
    `value` is the multi-threaded decode rate."""
    from threadpoolctl import threadpool_limits
    from oracle.attention import reference_outputs
    from oracle.episode import run_episode
    from prefix_shared_kv_radix_amd.runner import Engine
    w.kv_table()
    w.q_table()   # built once, outside every timed sample
    t0 = time.perf_counter()
    log = run_episode(w)
    t_py = time.perf_counter() - t0
    t0 = time.perf_counter()
    Engine(w).run()
    t_cpp = time.perf_counter() - t0
    threads = _oracle_threads()
    n, dt, ctx = _decode_queries(w, log, seconds)
    with threadpool_limits(1):
        n1, dt1, _ = _decode_queries(w, log, seconds / 4)
    ext = [a for rnd in log.rounds for a in rnd.admissions
           if w.phases[rnd.phase].extend == "attend" and a.prompt_len > a.prefix_len]
    ext_rate, ext_desc = None, "none"
    if ext:
        a = ext[-1]
        pos = np.arange(a.prefix_len, a.prompt_len)
        t0 = time.perf_counter()
        reference_outputs(w, a.rid, pos)
        te = time.perf_counter() - t0
        ext_rate = len(pos) / te
        ext_desc = f"{len(pos)} rows on a {a.prefix_len}-token prefix in {te:.2f}s"
    return {"value": n / dt, "unit": "decode tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} decode queries (from step 0 on, L~{ctx}) of {w.name} in {dt:.1f}s, "
                      f"fp64 exact attention, {threads} BLAS threads",
            "single_thread": {"value": n1 / dt1, "unit": "decode tokens/s",
                              "sample": f"{n1} decode queries in {dt1:.1f}s on one thread"},
            "extend": {"value": ext_rate, "unit": "extend tokens/s", "sample": ext_desc},
            "host_tree": {"python_oracle_s": t_py, "cpp_library_s": t_cpp,
                          "speedup": t_py / t_cpp if t_cpp > 0 else None,
                          "sample": f"one {w.name} episode: admit (match, pin, alloc with "
                                    f"eviction), schedule, decode-slot allocation, insert"},
            "host_cores_visible": len(os.sched_getaffinity(0))}


def read_bandwidth(mib=1024, reps=10):
    """Device read rate of the library's streaming read probe (radix_probe_read) over
    `mib` MiB (bytes read per second, median of `reps` event-timed passes on the current
    stream): the practical read-only ceiling beside the nominal 8 TB/s."""
    import torch
    from prefix_shared_kv_radix_amd import _lib
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    _lib.probe_read(x, sink)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        _lib.probe_read(x, sink)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    del x, sink
    return 4.0 * n / float(np.median(times)) / 1e9


def copy_bandwidth(mib=1024, reps=10):
    """Device-to-device copy rate (read + write bytes per second) of a plain copy of
    `mib` MiB, median of `reps` event-timed copies: the practical HBM ceiling next to
    the nominal 8 TB/s."""
    import torch
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    y.copy_(x)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        y.copy_(x)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    del x, y
    return 2.0 * n / float(np.median(times)) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requests shard across GPUs with no exchange inside attention); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from prefix_shared_kv_radix_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n}))
        return
    w = workload_of(args.config)
    if args.layers < 1:
        print("--layers must be at least 1", file=sys.stderr)
        sys.exit(2)
    ep = Episode(w, not args.no_plan, args.splits, args.layers, args.schedule, args.ahead,
                 args.min_members, args.split_keys)
    torch.cuda.synchronize()
    print(f"[bench] staged {w.name}: {len(ep.rounds)} rounds", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        ep.run()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    # timed region: K steps with only three events per round (the extend/decode split)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ep.run(mark=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] timed {args.steps} steps in {t1 - t0:.3f}s", file=sys.stderr, flush=True)
    # the same K steps again with a HIP event pair around every launch (per-kernel
    # durations for the roofline); kept out of the region above because the per-launch
    # events cost the step several percent
    prof = []
    if not args.no_kernel_timing:
        _lib.profile_enable(1 << 17)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ep.run()
        torch.cuda.synchronize()
        prof = _lib.profile_read(1 << 17)
        _lib.profile_enable(0)
        print(f"[bench] kernel-timed {args.steps} more steps", file=sys.stderr, flush=True)

    # every figure below is per attention layer: an episode runs `layers` of them
    L = args.layers
    ms_per_step = (t1 - t0) * 1e3 / args.steps / L
    dec_tokens = sum(st["B"] * st["ph"].n_decode for st in ep.staged)
    ext_tokens = sum(st["T"] for st in ep.staged if st["ph"].extend == "attend")
    ext_ms = dec_ms = 0.0
    for seq in ep.marks:
        for i in range(0, len(seq), 3):
            ext_ms += seq[i][1].elapsed_time(seq[i + 1][1])
            dec_ms += seq[i + 1][1].elapsed_time(seq[i + 2][1])
    ext_ms /= args.steps * L
    dec_ms /= args.steps * L
    kern = {}
    for name, t in prof:
        k = kern.setdefault(name, [0, 0.0])
        k[0] += 1
        k[1] += t
    kernels = {n: {"launches": c // (args.steps * L), "ms_per_step": t / (args.steps * L),
                   "avg_us": 1e3 * t / c}
               for n, (c, t) in kern.items()}
    if not kern:   # no kernel-timed pass: phase times only
        out = {"metric": "decode tokens/s + achieved HBM GB/s (% peak), prefix-shared KV attention",
               "value": dec_tokens / (ms_per_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
               "extend_ms_per_step": ext_ms, "decode_ms_per_step": dec_ms,
               "config": {"workload": w.name, "layers": L, "schedule": args.schedule}}
        print(json.dumps(out))
        return
    dom = max(kern, key=lambda n: kern[n][1])
    byt, flop = algorithmic(w, ep, dom)
    t_dom = kern[dom][1] / (args.steps * L) / 1e3    # seconds per layer-episode in that kernel
    if dom in ("extend_mfma", "mla_decode"):   # dense bf16 contractions: MFMA-bound
        roof = {"bound": "mfma", "achieved": flop / t_dom / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byt / t_dom / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    copy_gbps = copy_bandwidth()
    read_gbps = read_bandwidth()
    if roof["bound"] == "hbm":
        roof["copy_gbps"] = copy_gbps
        roof["frac_of_copy"] = roof["achieved"] / copy_gbps
        roof["read_gbps"] = read_gbps
        roof["frac_of_read"] = roof["achieved"] / read_gbps
    roof["kernel"] = dom
    roof["avg_launch_us"] = 1e3 * kern[dom][1] / kern[dom][0]
    roof["algorithmic_bytes_per_launch"] = byt / (kern[dom][0] / (args.steps * L))
    roof["traffic"] = measured_traffic(dom, w.name)
    roof["sources"] = kernel_sources_digest()
    # decode-phase aggregate HBM rate over all decode kernels' algorithmic bytes
    dec_bytes = sum(algorithmic(w, ep, n)[0] for n in ("decode_tail_valu", "segment_mfma",
                                                         "decode_fused", "mla_decode") if n in kern)
    ext_flops = algorithmic(w, ep, "extend_mfma")[1]
    out = {
        "metric": "decode tokens/s + achieved HBM GB/s (% peak), prefix-shared KV attention",
        "value": dec_tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.shape.kv_dtype if w.shape.kv_dtype != "fp8" else "fp8-kv/bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pool_slots": w.pool_slots,
                   "q_heads": w.shape.num_q_heads, "kv_heads": w.shape.num_kv_heads,
                   "head_dim": w.shape.head_dim_qk, "decode_tokens_per_step": dec_tokens,
                   "extend_tokens_per_step": ext_tokens, "shared_segments": not args.no_plan,
                   "layers": L, "schedule": args.schedule,
                   "ahead": args.ahead if args.schedule == "overlap" else None},
        "extend_ms_per_step": ext_ms,
        "decode_ms_per_step": dec_ms,
        "decode_only_tokens_per_s": dec_tokens / (dec_ms / 1e3) if dec_ms else None,
        "extend_tokens_per_s": ext_tokens / (ext_ms / 1e3) if ext_ms else None,
        "extend_tflops": ext_flops / (ext_ms / 1e3) / 1e12 if ext_ms else None,
        "decode_algorithmic_gbps": dec_bytes / (dec_ms / 1e3) / 1e9 if dec_ms else None,
        "decode_hbm_frac_of_peak": dec_bytes / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBPS if dec_ms else None,
        "copy_gbps": copy_gbps,
        "read_gbps": read_gbps,
        "extend_mfma_frac_of_peak": ext_flops / (ext_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS if ext_ms else None,
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
