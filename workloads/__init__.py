"""Seeded synthetic inputs for the radix-shared KV attention path.

This module only draws random numbers and lays out request scripts. It holds
none of the method's arithmetic: no prefix matching, no slot assignment, no
eviction and no attention. Both the CPU oracle (``oracle/``) and the HIP path
(``prefix_shared_kv_radix_amd``) consume what it produces.

Workload shapes follow the sharing patterns described on the page
"49 · RadixAttention, eviction và cache churn" (§1 layered sharing: a system
prompt with few-shot examples then different questions, a chat growing turn by
turn, an agent forking many attempts from one point; §6 cyclic prefixes through
a cache of four) and the MLA decode shape of the SGLang feature article (§一,
one latent KV head read by many query heads).

Conventions
-----------
* Token ids are uniform on [0, 32000) (``numpy`` PCG64, seeded per config).
  Where a request branches off a shared path, its first divergent token is
  redrawn until it differs from every sibling's, so the designed tree shape
  is exactly the one the token ids produce.
* Every token position of every request carries a *content id* (``kv_ids``).
  Two requests that share a token prefix share the content ids of that prefix,
  because a causal model's K/V of a prefix depends only on the prefix. The K/V
  row of a content id is row ``id % table_rows`` of a seeded N(0, 1) table.
* Query rows are drawn from a seeded N(0, 1) table as well: the query of
  request ``rid`` at absolute position ``pos`` is row
  ``(rid * 1000003 + pos * 7919) % q_rows``.
* Values are rounded to the I/O dtype once, here; both sides read the same
  rounded values. bf16 is stored as its 16-bit pattern (``uint16``), fp8 E4M3
  as its byte (``uint8``) plus one fp32 scale per token row.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

VOCAB = 32000
Q_ROW_MUL = 1000003
Q_POS_MUL = 7919


# --------------------------------------------------------------------------
# value rounding helpers (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns uint16 bit patterns.
    Works through the values in chunks (64-bit temporaries of a whole table would take
    several times its size)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    fu, fo = u.reshape(-1), out.reshape(-1)
    step = 1 << 20
    for i in range(0, fu.size, step):
        c = fu[i:i + step].astype(np.uint64)
        c += 0x7FFF + ((c >> 16) & 1)
        c >>= 16
        fo[i:i + step] = c
    return out


def quantize_e4m3_rows(x: np.ndarray):
    """Per-row fp8 E4M3 (OCP 'fn' variant) quantisation for test data.

    scale = amax(|row|) / 448 (1 where the row is all zero); bytes = RNE(row / scale).
    Uses torch's CPU cast, which rounds to nearest even; |row / scale| <= 448 so
    nothing saturates. Returns (uint8 bytes with x's shape, float32 scale [rows]).
    """
    import torch

    rows = x.shape[0]
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(rows, -1)
    amax = np.abs(flat).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    t = torch.from_numpy(flat / scale[:, None])
    q = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q.reshape(x.shape).copy(), scale


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    q_dtype: str            # 'f32' | 'bf16'   (also the output dtype)
    kv_dtype: str           # 'f32' | 'bf16' | 'fp8'
    v_is_k_prefix: bool     # MLA: V is the first head_dim_v dims of the K row
    sm_scale: float

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class Request:
    rid: int
    tokens: np.ndarray       # int32 [n] prompt token ids
    kv_ids: np.ndarray       # int64 [n] content id per prompt position
    out_tokens: np.ndarray   # int32 [n_out] tokens fed during decode (greedy-free)
    out_kv_ids: np.ndarray   # int64 [n_out]


@dataclass
class Phase:
    """A set of requests queued together.

    Rounds repeat until the queue is empty: order the queue by ``policy``,
    admit up to ``batch_limit`` requests, extend them as one batch, run
    ``n_decode`` decode steps on the admitted batch, then finish them all.
    ``extend`` says what device work the phase's extend does:
    'attend' (store new K/V and run extend attention), 'store' (store only),
    'host' (no device work; the harness fills the pool before the next
    device phase).
    """
    rids: List[int]
    policy: str = "fcfs"
    batch_limit: int = 1 << 30
    n_decode: int = 0
    extend: str = "attend"


@dataclass
class Workload:
    name: str
    seed: int
    shape: AttnShape
    pool_slots: int
    requests: List[Request]
    phases: List[Phase]
    n_kv_ids: int
    table_rows: int
    q_rows: int
    note: str = ""
    _cache: Dict[str, object] = field(default_factory=dict, repr=False)

    # ---- K/V table -------------------------------------------------------
    def kv_table(self):
        """Return (K, V, K_scale).

        K: [table_rows, Hkv, Dqk]; V: [table_rows, Hkv, Dv] or None when V is the
        K prefix (MLA). Storage dtype: float32 ('f32'), uint16 bf16 bits ('bf16'),
        uint8 E4M3 bytes ('fp8'). K_scale: float32 [table_rows] for fp8, else None.
        """
        if "kv" not in self._cache:
            s = self.shape
            rng = np.random.default_rng([self.seed, 1])
            k = _normal(rng, (self.table_rows, s.num_kv_heads, s.head_dim_qk))
            v = None
            if not s.v_is_k_prefix:
                rng_v = np.random.default_rng([self.seed, 2])
                v = _normal(rng_v, (self.table_rows, s.num_kv_heads, s.head_dim_v))
            scale = None
            if s.kv_dtype == "f32":
                pass
            elif s.kv_dtype == "bf16":
                k = f32_to_bf16_bits(k)
                v = None if v is None else f32_to_bf16_bits(v)
            elif s.kv_dtype == "fp8":
                if v is None:
                    k, scale = quantize_e4m3_rows(k)
                else:
                    # one scale per token: the token's K and V rows (all KV heads) together
                    kv, scale = quantize_e4m3_rows(np.concatenate([k, v], axis=-1))
                    k = np.ascontiguousarray(kv[..., :s.head_dim_qk])
                    v = np.ascontiguousarray(kv[..., s.head_dim_qk:])
            else:
                raise ValueError(s.kv_dtype)
            self._cache["kv"] = (k, v, scale)
        return self._cache["kv"]

    def kv_rows(self, kv_ids: np.ndarray) -> np.ndarray:
        return (np.asarray(kv_ids, dtype=np.int64) % self.table_rows).astype(np.int64)

    # ---- query table -----------------------------------------------------
    def q_table(self) -> np.ndarray:
        """[q_rows, Hq, Dqk] in the query dtype's storage (float32 or uint16 bf16 bits)."""
        if "q" not in self._cache:
            s = self.shape
            rng = np.random.default_rng([self.seed, 3])
            q = _normal(rng, (self.q_rows, s.num_q_heads, s.head_dim_qk))
            if s.q_dtype == "bf16":
                q = f32_to_bf16_bits(q)
            self._cache["q"] = q
        return self._cache["q"]

    def q_index(self, rid: int, positions: np.ndarray) -> np.ndarray:
        pos = np.asarray(positions, dtype=np.int64)
        return (np.int64(rid) * Q_ROW_MUL + pos * Q_POS_MUL) % self.q_rows

    # ---- helpers ---------------------------------------------------------
    def full_tokens(self, rid: int) -> np.ndarray:
        r = self.requests[rid]
        return np.concatenate([r.tokens, r.out_tokens]).astype(np.int32)

    def full_kv_ids(self, rid: int) -> np.ndarray:
        r = self.requests[rid]
        return np.concatenate([r.kv_ids, r.out_kv_ids]).astype(np.int64)


def _normal(rng, shape):
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        flat[i:i + step] = rng.standard_normal(min(step, flat.size - i), dtype=np.float32)
    return out


# --------------------------------------------------------------------------
# token drawing with distinct branch points
# --------------------------------------------------------------------------
class _Tokens:
    def __init__(self, seed: int):
        self.rng = np.random.default_rng([seed, 0])
        self.next_id = 0

    def draw(self, n: int, avoid_first: Optional[set] = None) -> np.ndarray:
        t = self.rng.integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32)
        if n and avoid_first is not None:
            while int(t[0]) in avoid_first:
                t[0] = int(self.rng.integers(0, VOCAB))
            avoid_first.add(int(t[0]))
        return t

    def ids(self, n: int) -> np.ndarray:
        out = np.arange(self.next_id, self.next_id + n, dtype=np.int64)
        self.next_id += n
        return out


def _req(rid, tokens, kv_ids, out_tokens=None, out_kv_ids=None):
    if out_tokens is None:
        out_tokens = np.zeros(0, np.int32)
        out_kv_ids = np.zeros(0, np.int64)
    return Request(rid, np.asarray(tokens, np.int32), np.asarray(kv_ids, np.int64),
                   np.asarray(out_tokens, np.int32), np.asarray(out_kv_ids, np.int64))


# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------
def tiny_shape() -> AttnShape:
    return AttnShape(4, 4, 64, 64, "f32", "f32", False, 1.0 / 8.0)


def gqa128_shape(kv_dtype: str = "bf16") -> AttnShape:
    """Llama-3-8B attention shape: 32 query heads, 8 KV heads, head dim 128, bf16 queries;
    K/V bf16, or fp8 E4M3 with one scale per token."""
    return AttnShape(32, 8, 128, 128, "bf16", kv_dtype, False, 1.0 / math.sqrt(128.0))


def mla_shape(kv_dtype: str = "bf16") -> AttnShape:
    """DeepSeek-V3 MLA decode shape: 128 query heads, one latent KV head of 512 + 64 rope dims."""
    return AttnShape(128, 1, 576, 512, "bf16", kv_dtype, True, 1.0 / math.sqrt(576.0))


# --------------------------------------------------------------------------
# workload builders
# --------------------------------------------------------------------------
def few_shot(seed: int, shape: AttnShape, prefix_len: int, n_req: int, q_len: int,
             n_decode: int, pool_slots: Optional[int] = None, name: str = "few_shot",
             q_rows: int = 16384) -> Workload:
    """One warm request holding a shared prefix, then ``n_req`` requests = prefix + a
    unique ``q_len``-token question, extended as one batch and decoded ``n_decode`` steps."""
    g = _Tokens(seed)
    prefix = g.draw(prefix_len)
    prefix_ids = g.ids(prefix_len)
    reqs = [_req(0, prefix, prefix_ids)]
    firsts: set = set()
    for r in range(1, n_req + 1):
        q = g.draw(q_len, firsts)
        reqs.append(_req(r, np.concatenate([prefix, q]), np.concatenate([prefix_ids, g.ids(q_len)])))
    for r in range(1, n_req + 1):
        reqs[r].out_tokens = g.draw(n_decode)
        reqs[r].out_kv_ids = g.ids(n_decode)
    if pool_slots is None:
        pool_slots = prefix_len + n_req * (q_len + n_decode)
    phases = [Phase([0], "fcfs", 1, 0, "attend"),
              Phase(list(range(1, n_req + 1)), "fcfs", n_req, n_decode, "attend")]
    return Workload(name, seed, shape, pool_slots, reqs, phases, g.next_id, g.next_id,
                    q_rows)


def chat_tree(seed: int, shape: AttnShape, n_conv: int, n_turns: int, turn_lo: int,
              turn_hi: int, pool_frac: float = 0.7, name: str = "chat_tree",
              q_rows: int = 16384) -> Workload:
    """Multi-turn chat: turn t of every conversation is a request whose prompt is the
    conversation's turns 0..t; turns are served round-robin (all turn t, then t+1).
    Pool = ceil(pool_frac x all distinct tokens), so history gets evicted and
    recomputed."""
    g = _Tokens(seed)
    firsts: set = set()
    conv_tok, conv_ids, lens = [], [], []
    for c in range(n_conv):
        tl = g.rng.integers(turn_lo, turn_hi + 1, size=n_turns)
        toks = [g.draw(int(tl[0]), firsts)] + [g.draw(int(n)) for n in tl[1:]]
        conv_tok.append(np.concatenate(toks))
        conv_ids.append(g.ids(int(tl.sum())))
        lens.append(np.cumsum(tl))
    reqs, phases = [], []
    for t in range(n_turns):
        rids = []
        for c in range(n_conv):
            n = int(lens[c][t])
            rid = len(reqs)
            reqs.append(_req(rid, conv_tok[c][:n], conv_ids[c][:n]))
            rids.append(rid)
        phases.append(Phase(rids, "fcfs", n_conv, 0, "attend"))
    total = int(sum(len(x) for x in conv_tok))
    pool = int(math.ceil(pool_frac * total))
    return Workload(name, seed, shape, pool, reqs, phases, g.next_id, g.next_id, q_rows,
                    note=f"{total} distinct tokens, pool {pool}")


def chat_decode(seed: int, shape: AttnShape, n_dec: int, ctx_lo: int, ctx_hi: int,
                turn_lo: int, turn_hi: int, n_decode: int, bg_turns: int = 8,
                pool_factor: float = 1.05, ws_frac: float = 0.7, batch_limit: int = 512,
                table_rows: Optional[int] = None, name: str = "chat_decode",
                q_rows: int = 16384) -> Workload:
    """Decode batch over long chat histories whose slots were scattered by churn.

    ``n_dec`` conversations grow turn by turn to a target context ~ U[ctx_lo, ctx_hi];
    background conversations of ``bg_turns`` turns are interleaved round-robin with
    them. Pool = ceil(pool_factor x (sum of targets + n_dec x n_decode)); the
    background volume makes the pool about ``ws_frac`` of all distinct tokens.
    History phases are host-only; the last phase admits all ``n_dec`` full
    histories at once (re-extending evicted parts) and decodes ``n_decode`` steps."""
    g = _Tokens(seed)
    firsts: set = set()
    ctx = g.rng.integers(ctx_lo, ctx_hi + 1, size=n_dec)
    pool = int(math.ceil(pool_factor * (int(ctx.sum()) + n_dec * n_decode)))
    bg_total_target = max(0, int(pool / ws_frac) - int(ctx.sum()))
    convs = []   # (tokens, ids, cumulative turn ends)
    for c in range(n_dec):
        ends, tot = [], 0
        while tot < ctx[c]:
            tot = min(int(ctx[c]), tot + int(g.rng.integers(turn_lo, turn_hi + 1)))
            ends.append(tot)
        toks = g.draw(int(ctx[c]), firsts)
        convs.append((toks, g.ids(int(ctx[c])), ends))
    bg_total = 0
    while bg_total < bg_total_target:
        tl = g.rng.integers(turn_lo, turn_hi + 1, size=bg_turns)
        n = int(tl.sum())
        toks = g.draw(n, firsts)
        convs.append((toks, g.ids(n), list(np.cumsum(tl))))
        bg_total += n
    reqs, phases = [], []
    max_turns = max(len(c[2]) for c in convs)
    for t in range(max_turns):
        rids = []
        for c, (toks, ids, ends) in enumerate(convs):
            # the decode conversations' last turn is served by the final phase
            last = len(ends) - 1 if c >= n_dec else len(ends) - 2
            if t <= last:
                n = int(ends[t])
                rid = len(reqs)
                reqs.append(_req(rid, toks[:n], ids[:n]))
                rids.append(rid)
        if rids:
            phases.append(Phase(rids, "fcfs", batch_limit, 0, "host"))
    final = []
    for c in range(n_dec):
        toks, ids, _ = convs[c]
        rid = len(reqs)
        reqs.append(_req(rid, toks, ids, g.draw(n_decode), g.ids(n_decode)))
        final.append(rid)
    phases.append(Phase(final, "fcfs", n_dec, n_decode, "attend"))
    if table_rows is None:
        table_rows = g.next_id
    return Workload(name, seed, shape, pool, reqs, phases, g.next_id, min(table_rows, g.next_id),
                    q_rows, note=f"decode contexts sum {int(ctx.sum())}, background {bg_total}, pool {pool}")


def agent_branch(seed: int, shape: AttnShape, n_roots: int, root_len: int, branches: int,
                 branch_len: int, forks: int, n_decode: int, name: str = "agent_branch",
                 q_rows: int = 16384) -> Workload:
    """Agent branching: roots (prefill, no prefix), branches forking off each root
    (extend on the cached root), then ``forks`` decode samples per branch."""
    g = _Tokens(seed)
    root_first: set = set()
    reqs, roots, brs, dec = [], [], [], []
    root_tok = []
    for r in range(n_roots):
        t, ids = g.draw(root_len, root_first), g.ids(root_len)
        root_tok.append((t, ids))
        roots.append(len(reqs))
        reqs.append(_req(len(reqs), t, ids))
    br_tok = []
    for r in range(n_roots):
        firsts: set = set()
        for b in range(branches):
            t = np.concatenate([root_tok[r][0], g.draw(branch_len, firsts)])
            ids = np.concatenate([root_tok[r][1], g.ids(branch_len)])
            br_tok.append((t, ids))
            brs.append(len(reqs))
            reqs.append(_req(len(reqs), t, ids))
    for t, ids in br_tok:
        firsts = set()
        for f in range(forks):
            out = g.draw(n_decode, firsts)
            dec.append(len(reqs))
            reqs.append(_req(len(reqs), t, ids, out, g.ids(n_decode)))
    pool = n_roots * root_len + n_roots * branches * branch_len + len(dec) * n_decode
    phases = [Phase(roots, "fcfs", len(roots), 0, "attend"),
              Phase(brs, "fcfs", len(brs), 0, "attend"),
              Phase(dec, "fcfs", len(dec), n_decode, "attend")]
    return Workload(name, seed, shape, pool, reqs, phases, g.next_id, g.next_id, q_rows)


def cyclic_stream(seed: int, shape: AttnShape, n_prefixes: int = 5, prefix_len: int = 2048,
                  cycles: int = 2, cache_prefixes: int = 4, order: str = "cyclic",
                  policy: str = "fcfs", extend: str = "attend", name: str = "cyclic",
                  q_rows: int = 16384) -> Workload:
    """Cyclic prefix stream (page 4 §6): ``n_prefixes`` distinct prefixes arrive in
    the order A, B, C, ... repeated ``cycles`` times ('cyclic') or the same traffic
    grouped per prefix A, A, B, B, ... ('grouped'); the pool holds exactly
    ``cache_prefixes`` prefixes; one request per round; all requests are queued at once."""
    g = _Tokens(seed)
    firsts: set = set()
    pre = [(g.draw(prefix_len, firsts), g.ids(prefix_len)) for _ in range(n_prefixes)]
    if order == "cyclic":
        seq = [p for _ in range(cycles) for p in range(n_prefixes)]
    elif order == "grouped":
        seq = [p for p in range(n_prefixes) for _ in range(cycles)]
    else:
        raise ValueError(order)
    reqs = [_req(i, pre[p][0], pre[p][1]) for i, p in enumerate(seq)]
    phases = [Phase(list(range(len(reqs))), policy, 1, 0, extend)]
    return Workload(name, seed, shape, cache_prefixes * prefix_len, reqs, phases, g.next_id,
                    g.next_id, q_rows, note=f"order={order} policy={policy}")


def mla_groups(seed: int, kv_dtype: str, n_groups: int, group_len: int, per_group: int,
               unique_len: int, n_decode: int, name: str = "mla_groups",
               q_rows: int = 4096) -> Workload:
    """MLA decode: ``n_groups`` radix-shared prefixes, ``per_group`` requests each with
    a unique continuation; the pool rows of the prompts are stored directly (no MLA
    extend attention), then ``n_decode`` decode steps at full batch."""
    shape = mla_shape(kv_dtype)
    g = _Tokens(seed)
    gfirst: set = set()
    reqs, heads, members = [], [], []
    gp = []
    for i in range(n_groups):
        t, ids = g.draw(group_len, gfirst), g.ids(group_len)
        gp.append((t, ids))
        heads.append(len(reqs))
        reqs.append(_req(len(reqs), t, ids))
    for i in range(n_groups):
        firsts: set = set()
        for j in range(per_group):
            t = np.concatenate([gp[i][0], g.draw(unique_len, firsts)])
            ids = np.concatenate([gp[i][1], g.ids(unique_len)])
            members.append(len(reqs))
            reqs.append(_req(len(reqs), t, ids))
    # members are listed group by group; interleave arrival order across groups so
    # grouping comes from the tree rather than from request order
    order = [members[i * per_group + j] for j in range(per_group) for i in range(n_groups)]
    for rid in members:
        reqs[rid].out_tokens = g.draw(n_decode)
        reqs[rid].out_kv_ids = g.ids(n_decode)
    pool = n_groups * group_len + len(members) * (unique_len + n_decode)
    phases = [Phase(heads, "fcfs", len(heads), 0, "store"),
              Phase(order, "fcfs", len(order), n_decode, "store")]
    return Workload(name, seed, shape, pool, reqs, phases, g.next_id, g.next_id, q_rows)


def mixed_hits(seed: int, shape: AttnShape, base_len: int, ext_len: int, n_decode: int,
               name: str = "mixed_hits", q_rows: int = 4096) -> Workload:
    """An extend batch mixing fully cached prompts (nothing to extend) with partly
    cached and uncached ones. Warm phase: prompts A (``base_len`` tokens) and
    B = A + ``ext_len`` tokens. Then one batch of: A again, B again (both wholly
    cached), A + a new continuation, B + a new continuation and an unrelated prompt,
    each decoded ``n_decode`` steps."""
    g = _Tokens(seed)
    a_tok, a_ids = g.draw(base_len, set()), g.ids(base_len)
    firsts: set = set()
    b_more = g.draw(ext_len, firsts)
    b_tok, b_ids = np.concatenate([a_tok, b_more]), np.concatenate([a_ids, g.ids(ext_len)])
    reqs = [_req(0, a_tok, a_ids), _req(1, b_tok, b_ids)]
    a_more = g.draw(ext_len // 2 + 3, firsts)
    prompts = [(a_tok, a_ids), (b_tok, b_ids),
               (np.concatenate([a_tok, a_more]), np.concatenate([a_ids, g.ids(len(a_more))])),
               (np.concatenate([b_tok, g.draw(ext_len + 5)]), np.concatenate([b_ids, g.ids(ext_len + 5)]))]
    other = g.draw(base_len // 2 + 7, {int(a_tok[0])})
    prompts.append((other, g.ids(len(other))))
    for t, ids in prompts:
        reqs.append(_req(len(reqs), t, ids, g.draw(n_decode), g.ids(n_decode)))
    pool = sum(len(r.tokens) for r in reqs) + len(prompts) * n_decode
    phases = [Phase([0, 1], "fcfs", 1, 0, "attend"),
              Phase(list(range(2, len(reqs))), "fcfs", len(prompts), n_decode, "attend")]
    return Workload(name, seed, shape, pool, reqs, phases, g.next_id, g.next_id, q_rows)


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "few_shot_gqa128",
    3: "multi_turn_chat",
    4: "agent_branching",
    5: "mla_decode",
}


def config(n: int, variant: str = "") -> Workload:
    """Full-size workload for configuration ``n`` (seed = n).

    variant: for 2, '' (bf16 K/V) or 'fp8' (E4M3 K/V, one scale per token);
    for 3, 'A' (chat tree extend under churn) or 'B' (scattered decode);
    for 4, '' (branching), 'fp8' (branching, E4M3 K/V), 'cyclic', 'grouped' or 'cyclic_lpf';
    for 5, 'bf16' or 'fp8'.
    """
    if n == 1:
        return few_shot(1, tiny_shape(), 64, 8, 32, 16, pool_slots=1024, name="tiny_fp32",
                        q_rows=1024)
    if n == 2:
        kv = variant or "bf16"
        return few_shot(2, gqa128_shape(kv), 2048, 256, 128, 128, pool_slots=67584,
                        name="few_shot_gqa128" + ("" if kv == "bf16" else "_fp8"))
    if n == 3:
        if variant in ("", "A"):
            return chat_tree(3, gqa128_shape(), 64, 8, 64, 256, 0.7, name="chat_tree_3A")
        if variant == "B":
            return chat_decode(3, gqa128_shape(), 256, 1024, 8192, 64, 256, 32,
                               table_rows=1 << 18, name="chat_decode_3B")
        raise ValueError(variant)
    if n == 4:
        if variant in ("", "fp8"):
            kv = variant or "bf16"
            return agent_branch(4, gqa128_shape(kv), 16, 4096, 8, 512, 4, 256,
                                name="agent_branch_4" + ("" if kv == "bf16" else "_fp8"))
        order, policy = {"cyclic": ("cyclic", "fcfs"), "grouped": ("grouped", "fcfs"),
                         "cyclic_lpf": ("cyclic", "lpf")}[variant]
        return cyclic_stream(4, gqa128_shape(), 5, 2048, 2, 4, order, policy,
                             name=f"cyclic_4_{variant}")
    if n == 5:
        kv = variant or "bf16"
        return mla_groups(5, kv, 8, 2048, 32, 2048, 32, name=f"mla_5_{kv}")
    raise ValueError(n)
