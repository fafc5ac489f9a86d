"""HIP path vs the CPU oracle, element by element, through the C ABI.

Each case runs a workload's request script through the native tree and the
gfx950 kernels (extend, shared-segment decode, split-KV decode, combine) and
compares the outputs with the oracle's exact attention over each request's
own keys (fp64): max-abs <= 1e-4 for fp32, <= 2e-2 for bf16 I/O with fp32
accumulation; LSE within 1e-5 / 1e-3.

fp8 K/V (E4M3 bytes times a per-token scale): the GQA extend and shared-segment
tiles round each dequantised element to a bf16 MMA operand (round to nearest even,
relative error at most 2^-8), so a score moves by at most
delta_j = sm_scale * sum_i |q_i k_ji| * 2^-8 (k_j of the row's own KV head) and the
LSE, a smooth maximum of the scores, by at most delta = max_j delta_j over the keys
it sees. Each probability then changes by a factor within [e^-2delta, e^2delta] and
each value element by at most 2^-8 of itself, so output element d moves by at most
((e^2delta - 1)(1 + 2^-8) + 2^-8) * sum_j p_j |v_jd| (p the exact probabilities).
A GQA fp8 row's tolerances are these bounds, computed from the row's own query and
dequantised keys and values, on top of the bf16 tolerances. The MLA kernel converts
E4M3 to bf16 exactly and applies each key's scale to its score and probability, so
its fp8 rows get the bf16 tolerances alone.

Decode checks are gathered while the episode runs and computed afterwards, one
oracle call per request for all its checked positions, on a thread pool.
"""
import numpy as np
import pytest

from conftest import gpu_available
from oracle.attention import reference_outputs, request_kv, request_q
from workloads import (agent_branch, chat_decode, chat_tree, config, few_shot, gqa128_shape,
                       mixed_hits, tiny_shape)

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-5), "bf16": (2e-2, 1e-3)}
BF16_REL = 2.0 ** -8     # bf16 round-to-nearest-even relative error bound


def _to_np(t):
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def fp8_bounds(w, rid, positions):
    """Rounding bounds of GQA fp8 rows (see above): output [n, Hq, Dv] and LSE [n, Hq]
    for the request's queries at ``positions``, each head against its own KV head."""
    positions = np.asarray(positions, dtype=np.int64)
    L = int(positions.max()) + 1
    k, v = request_kv(w, w.full_kv_ids(rid)[:L])                 # [L, Hkv, Dqk], [L, Hkv, Dv]
    q = request_q(w, rid, positions)                              # [n, Hq, Dqk]
    n, hq, d = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    g = hq // hkv
    qk = q.reshape(n, hkv, g, d).transpose(1, 0, 2, 3).reshape(hkv, n * g, d)
    kt = k.transpose(1, 2, 0)                                     # [Hkv, Dqk, L]
    vis = (np.arange(L)[None, :] <= np.repeat(positions, g)[:, None])[None]
    delta = w.shape.sm_scale * BF16_REL * 1.01 * np.where(vis, np.abs(qk) @ np.abs(kt), 0.0).max(axis=2)
    s = np.where(vis, w.shape.sm_scale * (qk @ kt), -np.inf)
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    mean_abs_v = p @ np.abs(v).transpose(1, 0, 2)                 # [Hkv, n*G, Dv]
    out = (np.expm1(2.0 * delta) * (1.0 + BF16_REL) + BF16_REL)[..., None] * mean_abs_v
    out = out.reshape(hkv, n, g, dv).transpose(1, 0, 2, 3).reshape(n, hq, dv)
    lse = delta.reshape(hkv, n, g).transpose(1, 0, 2).reshape(n, hq)
    return out, lse


class Checker:
    """Collects device outputs through the runner's callbacks and checks them against
    the oracle: extend samples at once, decode outputs after the episode."""

    def __init__(self, w, extend_sample=None, decode_steps=None, decode_sample=None, seed=0):
        self.w = w
        self.rng = np.random.default_rng(seed)
        self.extend_sample = extend_sample
        self.decode_steps = decode_steps
        self.decode_sample = decode_sample
        self.tol_o, self.tol_l = TOL[w.shape.q_dtype]
        # MLA converts E4M3 exactly and scales scores and probabilities: the bf16 LSE
        # tolerance alone; GQA fp8 tiles round (value x scale) to bf16: add the bound
        self.fp8 = w.shape.kv_dtype == "fp8" and not w.shape.v_is_k_prefix
        self.worst = 0.0
        self.checked = 0
        self.pending = {}   # rid -> [(position, o, lse)]

    def _pick(self, n, k):
        if k is None or k >= n:
            return np.arange(n)
        return np.sort(self.rng.choice(n, size=k, replace=False))

    def _cmp(self, rid, pos, o, l, ref_o, ref_l, what):
        oerr = np.abs(o - ref_o)
        err = oerr.max()
        lerr = np.abs(l - ref_l)
        tol_o, tol_l = self.tol_o, self.tol_l
        if self.fp8:
            ob, lb = fp8_bounds(self.w, rid, pos)
            tol_o, tol_l = self.tol_o + ob, self.tol_l + lb
        self.worst = max(self.worst, err)
        self.checked += 1
        assert np.all(oerr <= tol_o), f"{what}: output max-abs {err} (bound {np.min(tol_o)})"
        assert np.all(lerr <= tol_l), f"{what}: lse max-abs {lerr.max()} (bound {np.min(tol_l)})"

    def on_extend(self, rnd, out, lse, cu):
        if out is None:
            return
        o_all, l_all = _to_np(out), _to_np(lse)
        for b in self._pick(len(rnd.admissions), self.extend_sample):
            a = rnd.admissions[b]
            if a.prompt_len == a.prefix_len:
                continue
            pos = np.arange(a.prefix_len, a.prompt_len)
            if len(pos) > 64:   # first, last and a random middle sample of positions
                pos = np.unique(np.concatenate([pos[:8], pos[-8:], self.rng.choice(pos, 24)]))
            ro, rl = reference_outputs(self.w, a.rid, pos)
            idx = cu[b] + (pos - a.prefix_len)
            self._cmp(a.rid, pos, o_all[idx], l_all[idx], ro, rl, f"extend rid {a.rid}")

    def on_decode(self, rnd, step, out, lse):
        if self.decode_steps is not None and step not in self.decode_steps:
            return
        o_all, l_all = _to_np(out), _to_np(lse)
        for b in self._pick(len(rnd.admissions), self.decode_sample):
            a = rnd.admissions[b]
            self.pending.setdefault(a.rid, []).append((a.prompt_len + step, o_all[b], l_all[b]))

    def finish(self):
        """Oracle for every gathered decode output (all of a request's positions in one
        call), on host threads."""
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        items = sorted(self.pending.items())
        self.pending = {}

        def one(item):
            rid, rows = item
            pos = np.array([p for p, _, _ in rows])
            ro, rl = reference_outputs(self.w, rid, pos)
            return rid, pos, rows, ro, rl

        with threadpool_limits(1), ThreadPoolExecutor(16) as ex:
            for rid, pos, rows, ro, rl in ex.map(one, items):
                o = np.stack([x[1] for x in rows])
                l = np.stack([x[2] for x in rows])
                self._cmp(rid, pos, o, l, ro, rl, f"decode rid {rid} positions {pos.tolist()}")


def _run(w, checker, **kw):
    import torch
    from prefix_shared_kv_radix_amd.runner import Engine
    print(f"[gpu case] {w.name} {kw}", flush=True)
    eng = Engine(w, device="cuda", on_extend=checker.on_extend, on_decode=checker.on_decode, **kw)
    log = eng.run()
    torch.cuda.synchronize()
    checker.finish()
    assert checker.checked > 0
    print(f"[gpu case] {w.name} ok: {checker.checked} checks, worst {checker.worst:.3g}", flush=True)
    return log


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("use_plan,splits", [(True, 0), (False, 1), (False, 3), (True, 2)])
def test_tiny_fp32_all_outputs(use_plan, splits):
    """Config 1 in full: every extend and decode output of every request."""
    w = config(1)
    _run(w, Checker(w), use_plan=use_plan, num_splits=splits)


@pytest.mark.parametrize("use_plan,splits", [(True, 0), (False, 1), (False, 5), (True, 3)])
def test_few_shot_bf16_small(use_plan, splits):
    """GQA-128 bf16, 300-token shared prefix, 24 requests x 37 new tokens (ragged MFMA
    tiles), 9 decode steps, all outputs."""
    w = few_shot(2, gqa128_shape(), 300, 24, 37, 9, q_rows=4096)
    _run(w, Checker(w), use_plan=use_plan, num_splits=splits)


def test_few_shot_bf16_late_private_chunks():
    """Private tails of 90+ keys: with the plan, the last tenth of the requests (3 of
    30) read theirs in two chunks while the others fold the shared partials into one;
    every output of every request."""
    w = few_shot(5, gqa128_shape(), 200, 30, 90, 4, q_rows=4096)
    _run(w, Checker(w))


@pytest.mark.parametrize("use_plan,splits", [(True, 0), (True, 3), (False, 0), (False, 4)])
def test_few_shot_bf16_one_token_tails(use_plan, splits):
    """One-token questions: the private tails hold 1 to 5 pool rows, so most rows of a
    tail wave's 16-row iteration are masked, and with 3 or 4 chunks most chunks are
    empty; every output of every request."""
    w = few_shot(6, gqa128_shape(), 200, 24, 1, 5, q_rows=4096)
    _run(w, Checker(w), use_plan=use_plan, num_splits=splits)


@pytest.mark.parametrize("use_plan,splits", [(True, 0), (False, 1), (False, 3)])
def test_few_shot_bf16_host_slots(use_plan, splits):
    """New decode slots read by the kernel from pinned host memory (no copy launch)."""
    w = few_shot(12, gqa128_shape(), 200, 20, 29, 6, q_rows=4096)
    _run(w, Checker(w), use_plan=use_plan, num_splits=splits, host_slots=True)


@pytest.mark.parametrize("split_keys", [16, 24])
def test_tiny_fp32_segment_chunks(split_keys):
    """The 64-token shared prefix cut into key chunks by the plan: 4 full chunks, or 3
    chunks of which the last is empty (chunk lengths round up to 16 keys)."""
    w = config(1)
    _run(w, Checker(w), split_keys=split_keys)


@pytest.mark.parametrize("split_keys", [40, 100])
def test_agent_segment_chunks_bf16(split_keys):
    """Roots of 200 tokens and branches of 70 cut into key chunks (lengths round up to
    64 keys, so split_keys 40 leaves an empty last root chunk); every chunk is its own
    partial in the in-kernel merge."""
    w = agent_branch(4, gqa128_shape(), 3, 200, 4, 70, 3, 6, q_rows=4096)
    _run(w, Checker(w, extend_sample=4), split_keys=split_keys)


@pytest.mark.parametrize("branch_len,split_keys", [(600, None), (250, None), (600, 192)])
def test_agent_long_narrow_branches_bf16(branch_len, split_keys):
    """Narrow shared segments (3 forks x 4 heads = 12 query rows, one wave of a block's
    four) of 4 to 10 64-key tiles, also cut into 192-key chunks, with ragged last tiles,
    against the oracle."""
    w = agent_branch(5, gqa128_shape(), 2, 128, 3, branch_len, 3, 4, q_rows=4096)
    _run(w, Checker(w, extend_sample=2), split_keys=split_keys)


def test_decode_rejects_pageable_new_slots():
    """A pageable host slot list is refused on the host (E_INVAL) before any launch. The
    call also has no workspace for its 3 key splits, so nothing could be launched even if
    the pointer check were missing: the error text tells which check answered."""
    import torch
    from prefix_shared_kv_radix_amd import _lib
    from prefix_shared_kv_radix_amd.runner import DeviceState
    w = few_shot(12, gqa128_shape(), 40, 2, 8, 1, q_rows=64)
    d = DeviceState(w, "cuda", 2, 64)
    s = w.shape
    B = 2
    q = torch.zeros((B, s.num_q_heads, s.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    kv_new = torch.zeros((B, s.num_kv_heads, s.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, s.num_q_heads, s.head_dim_v), dtype=torch.bfloat16, device="cuda")
    seq = d.i32([5, 5])
    pageable = torch.zeros(B, dtype=torch.int32)
    assert not pageable.is_pinned()
    with pytest.raises(_lib.RadixError, match="new_slots"):
        _lib.attn_decode(d.shape, d.kv, q, kv_new, kv_new, None, pageable, d.rtt, None, seq, B, 8,
                         None, 3, out, None, None)
    torch.cuda.synchronize()


def test_agent_two_level_segments_bf16():
    """Roots, branches and forks: decode reads two nested shared segments per request."""
    w = agent_branch(4, gqa128_shape(), 3, 200, 4, 70, 3, 6, q_rows=4096)
    _run(w, Checker(w, extend_sample=6))


def test_chat_tree_under_churn_bf16():
    """Multi-turn chat with a pool at 40% of the working set: evicted history is
    recomputed, slot lists are scattered."""
    w = chat_tree(13, gqa128_shape(), 10, 5, 20, 90, 0.4, q_rows=4096)
    _run(w, Checker(w, extend_sample=5))


def test_chat_decode_scattered_bf16():
    w = chat_decode(3, gqa128_shape(), 16, 300, 1500, 30, 120, 4, batch_limit=12, q_rows=4096)
    _run(w, Checker(w))


def test_tiny_shapes_gqa_groups_fp32():
    """Query-head groups 1, 2, 4, 8 on the fp32 path."""
    import dataclasses
    for hq, hkv in ((4, 4), (4, 2), (8, 2), (8, 1)):
        shape = dataclasses.replace(tiny_shape(), num_q_heads=hq, num_kv_heads=hkv)
        w = few_shot(7, shape, 45, 5, 13, 3, q_rows=256)
        _run(w, Checker(w))


def test_gqa_groups_bf16():
    import dataclasses
    for hq, hkv in ((8, 8), (16, 8), (64, 8)):
        shape = dataclasses.replace(gqa128_shape(), num_q_heads=hq)
        w = few_shot(8, shape, 130, 6, 21, 3, q_rows=512)
        _run(w, Checker(w))


def test_few_shot_full_size():
    """Config 2 at full size (2048-token prefix x 256 requests x 128 tokens, 128 decode
    steps at batch 256): every request, head and dim at the first and last decode step;
    sampled extend rows."""
    w = config(2)
    _run(w, Checker(w, extend_sample=6, decode_steps={0, 127}))


def test_agent_full_size():
    """Config 4: 16 roots x 4096 (prefill), 128 branches x 512, 512 forks decoding
    256 steps through two nested shared segments: every request at the first and last
    decode step."""
    w = config(4)
    _run(w, Checker(w, extend_sample=3, decode_steps={0, 255}))


def test_chat_tree_full_size_sampled():
    w = config(3, "A")
    _run(w, Checker(w, extend_sample=3))


def test_chat_decode_full_size():
    """Config 3B: 256 decode requests with 1k-8k contexts scattered by churn; more
    private-tail items than resident waves (the work queue): every request at the
    first and last decode step."""
    w = config(3, "B")
    _run(w, Checker(w, decode_steps={0, 31}))


@pytest.mark.parametrize("splits", [8, 11])
def test_tail_work_queue_bf16(splits):
    """No plan, forced key splits: 96 requests x 8 KV heads x 8 (or 11) chunks give
    6144 (8448) private-tail items, three to four times the waves resident at once, so
    most items are drawn from the work queue; three decode steps reuse one workspace
    (its ticket counters must be back at zero after each call). Every output."""
    w = few_shot(31, gqa128_shape(), 600, 96, 40, 3, q_rows=4096)
    _run(w, Checker(w), use_plan=False, num_splits=splits)


@pytest.mark.parametrize("splits", [0, 3])
def test_eight_heads_per_kv_head_no_plan_bf16(splits):
    """64 query heads over 8 KV heads (8 per KV head) without a plan: the private-tail
    kernel's 8-head variant, whole and split; every output."""
    import dataclasses
    shape = dataclasses.replace(gqa128_shape(), num_q_heads=64)
    w = few_shot(9, shape, 170, 10, 23, 3, q_rows=512)
    _run(w, Checker(w), use_plan=False, num_splits=splits)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extend_batch_with_fully_cached_prompts(dtype):
    """One extend batch holding two wholly cached prompts (nothing to extend), two
    partly cached ones and an uncached one; then decode. Every output."""
    w = mixed_hits(21, gqa128_shape() if dtype == "bf16" else tiny_shape(), 150, 40, 3)
    ext = {}

    def spy(rnd, out, lse, cu):
        ext["E"] = [a.prompt_len - a.prefix_len for a in rnd.admissions]
        chk.on_extend(rnd, out, lse, cu)

    chk = Checker(w)
    import torch
    from prefix_shared_kv_radix_amd.runner import Engine
    print(f"[gpu case] {w.name} {dtype}", flush=True)
    Engine(w, device="cuda", on_extend=spy, on_decode=chk.on_decode).run()
    torch.cuda.synchronize()
    chk.finish()
    assert 0 in ext["E"] and max(ext["E"]) > 0
    assert chk.checked > 0


@pytest.mark.parametrize("kv,hq,n_conv,lo,hi", [
    ("bf16", 32, 72, 200, 330), ("fp8", 32, 72, 200, 330), ("bf16", 8, 256, 240, 320),
    ("bf16", 16, 136, 200, 330), ("bf16", 64, 40, 200, 330), ("fp8", 64, 40, 200, 330)])
def test_extend_ragged_turns_many_tiles(kv, hq, n_conv, lo, hi):
    """Three chat turns with ragged turn lengths, 1, 2, 4 or 8 query heads per KV head,
    sized to about 9 row tiles of 256 rows per CU: the persistent eight-wave extend
    grid, each block running 13 to 16 steps of its walk (and skipping the empty last
    tiles of the shorter requests); every request's first, last and sampled middle
    rows."""
    import dataclasses
    shape = dataclasses.replace(gqa128_shape(kv), num_q_heads=hq)
    w = chat_tree(41, shape, n_conv, 3, lo, hi, pool_frac=1.0, q_rows=4096)
    _run(w, Checker(w))


@pytest.mark.parametrize("use_plan,splits", [(True, 0), (False, 1), (False, 3), (True, 2)])
def test_few_shot_fp8_kv_small(use_plan, splits):
    """GQA-128 with fp8 E4M3 K/V (one scale per token): extend tiles and shared-segment
    tiles stage the bytes and convert them (times the scale) to bf16; the private tails
    convert them exactly and apply the scale to score and probability. All outputs."""
    w = few_shot(32, gqa128_shape("fp8"), 300, 24, 37, 9, q_rows=4096)
    _run(w, Checker(w), use_plan=use_plan, num_splits=splits)


def test_agent_fp8_kv_segment_chunks():
    """fp8 K/V through two nested shared segments cut into key chunks."""
    w = agent_branch(33, gqa128_shape("fp8"), 3, 200, 4, 70, 3, 6, q_rows=4096)
    _run(w, Checker(w, extend_sample=6), split_keys=100)


@pytest.mark.parametrize("hq,use_plan", [(8, True), (16, False), (64, True), (64, False)])
def test_fp8_kv_head_groups(hq, use_plan):
    """fp8 K/V with 1, 2 and 8 query heads per KV head (8 heads: compiler-placed waits)."""
    import dataclasses
    shape = dataclasses.replace(gqa128_shape("fp8"), num_q_heads=hq)
    w = few_shot(34, shape, 130, 6, 21, 3, q_rows=512)
    _run(w, Checker(w), use_plan=use_plan)


def test_fp8_kv_tail_work_queue():
    """fp8 private tails drawn from the work queue (more items than resident waves)."""
    w = few_shot(35, gqa128_shape("fp8"), 600, 96, 40, 3, q_rows=4096)
    _run(w, Checker(w), use_plan=False, num_splits=8)


def test_fp8_kv_extend_with_fully_cached_prompts():
    w = mixed_hits(36, gqa128_shape("fp8"), 150, 40, 3)
    _run(w, Checker(w))


@pytest.mark.parametrize("n", [2, 4])
def test_fp8_kv_full_size(n):
    """Configs 2 and 4 with fp8 K/V: every request at the first and last decode step."""
    w = config(n, "fp8")
    last = {2: 127, 4: 255}[n]
    _run(w, Checker(w, extend_sample=3, decode_steps={0, last}))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mla_small(kv):
    """MLA decode (128 heads, one 576-dim latent KV head, V = first 512 dims): three
    radix-shared prefixes, six requests each, 4 decode steps, all outputs."""
    from workloads import mla_groups
    w = mla_groups(5, kv, 3, 150, 6, 90, 4, q_rows=512)
    _run(w, Checker(w))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mla_splits_and_no_plan(kv):
    """Small batch: keys split across blocks and merged by the LSE combine; also without
    the radix plan (no request grouping)."""
    from workloads import mla_groups
    w = mla_groups(6, kv, 2, 700, 2, 900, 3, q_rows=512)
    _run(w, Checker(w), num_splits=3)
    _run(w, Checker(w), use_plan=False)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mla_short_contexts(kv):
    """Contexts of one to three 32-key tiles, and key chunks that are empty, one ragged
    tile or exactly one tile: every branch of the tile pipeline's start and end (fp8:
    the staging prologue, the clamped slot fetch past the end, the conversion of a
    tile that is never read)."""
    from workloads import mla_groups
    for seed, args, splits in ((7, (2, 20, 3, 15, 3), (1, 2)),     # 36..38 keys
                               (8, (2, 40, 2, 30, 3), (1, 4)),     # 71..73 keys: 3 tiles; 4 chunks
                               (9, (1, 10, 2, 5, 2), (1, 3))):     # 16..17 keys
        w = mla_groups(seed, kv, *args, q_rows=256)
        for ns in splits:
            _run(w, Checker(w), num_splits=ns)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mla_full_size(kv):
    """Config 5: 256 requests x 4096 context (2048-token prefixes shared by groups of
    32), 32 decode steps: every request at the first and last step."""
    w = config(5, kv)
    _run(w, Checker(w, decode_steps={0, 31}))
