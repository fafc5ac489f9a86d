"""Pins of the oracle's attention and storage decoding.

The attention the path computes is plain causal softmax attention per request
over the request's own keys (page "49 · RadixAttention, eviction và cache
churn", §2: the shared part is reused, only the new part is computed, so the
numbers must equal recomputation without sharing). The pins below fix it by
closed forms, by a library routine (torch's scaled_dot_product_attention in
fp64 on the CPU), by fp32/fp64 agreement, and by the shared-equals-unshared
property over a real radix-tree episode.
"""
import numpy as np
import pytest
import torch

from oracle.attention import (attention, attention_via_pool, bf16_bits_to_float, decode_storage,
                              e4m3fn_to_float, reference_outputs, request_kv)
from oracle.episode import run_episode
from workloads import config, f32_to_bf16_bits, few_shot, gqa128_shape, quantize_e4m3_rows


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------- closed forms
def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(0)
    L, hq, hkv, d = 9, 4, 2, 8
    k = np.repeat(_rand(rng, 1, hkv, d), L, axis=0)
    v = _rand(rng, L, hkv, d)
    q = _rand(rng, 3, hq, d)
    pos = np.array([2, 5, 8])
    o, lse = attention(q, k, v, pos, 0.3)
    for i, p in enumerate(pos):
        for h in range(hq):
            np.testing.assert_allclose(o[i, h], v[:p + 1, h // 2].mean(axis=0), rtol=0, atol=1e-13)


def test_constant_values_and_single_key():
    rng = np.random.default_rng(1)
    L, hq, d = 7, 2, 5
    k = _rand(rng, L, 1, d)
    c = _rand(rng, d)
    v = np.broadcast_to(c, (L, 1, d)).copy()
    o, _ = attention(_rand(rng, 4, hq, d), k, v, np.array([0, 1, 3, 6]), 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)
    v = _rand(rng, L, 1, d)
    o, lse = attention(_rand(rng, 1, hq, d), k, v, np.array([0]), 1.0)   # sees key 0 only
    np.testing.assert_array_equal(o[0, 0], v[0, 0])


def test_zero_query_is_mean_and_lse_is_log_count():
    rng = np.random.default_rng(2)
    L, d = 33, 16
    k, v = _rand(rng, L, 1, d), _rand(rng, L, 1, d)
    o, lse = attention(np.zeros((2, 1, d)), k, v, np.array([10, 32]), 0.125)
    np.testing.assert_allclose(o[0, 0], v[:11, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(o[1, 0], v[:, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], np.log([11.0, 33.0]), atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(3)
    L, d = 20, 4
    k = np.zeros((L, 1, d))
    k[13, 0, 0] = 60.0
    v = _rand(rng, L, 1, d)
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    o, lse = attention(q, k, v, np.array([L - 1]), 1.0)
    np.testing.assert_allclose(o[0, 0], v[13, 0], rtol=0, atol=1e-23)
    np.testing.assert_allclose(lse[0, 0], 60.0 + np.log1p((L - 1) * np.exp(-60.0)), atol=1e-13)


def test_mask_excludes_future_keys():
    """Changing a key/value beyond the query's position must not change its output."""
    rng = np.random.default_rng(4)
    k, v, q = _rand(rng, 12, 2, 8), _rand(rng, 12, 2, 8), _rand(rng, 1, 2, 8)
    o1, _ = attention(q, k, v, np.array([6]), 0.5)
    k[7:] += 100.0
    v[7:] -= 50.0
    o2, _ = attention(q, k, v, np.array([6]), 0.5)
    np.testing.assert_array_equal(o1, o2)


# ------------------------------------------------------------- library routine
@pytest.mark.parametrize("hq,hkv,dqk,dv,P,E", [(4, 4, 64, 64, 0, 7), (8, 2, 16, 16, 13, 5),
                                                (6, 1, 24, 12, 30, 1), (4, 2, 8, 8, 0, 1)])
def test_matches_torch_sdpa_fp64(hq, hkv, dqk, dv, P, E):
    rng = np.random.default_rng(hq * 100 + P)
    L = P + E
    q, k, v = _rand(rng, E, hq, dqk), _rand(rng, L, hkv, dqk), _rand(rng, L, hkv, dv)
    if dv < dqk:        # MLA-like: V is the K prefix
        v = k[:, :, :dv].copy()
    pos = np.arange(P, P + E)
    scale = 1.0 / np.sqrt(dqk)
    o, _ = attention(q, k, v, pos, scale)
    g = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)                       # [hq, E, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_fp32_oracle_agrees_with_fp64():
    w = config(1)
    for rid in (1, 5, 8):
        pos = np.arange(64, 96 + 16)
        o64, l64 = reference_outputs(w, rid, pos, np.float64)
        o32, l32 = reference_outputs(w, rid, pos, np.float32)
        assert np.abs(o64 - o32).max() < 1e-5
        assert np.abs(l64 - l32).max() < 1e-5


# ------------------------------------------------- shared equals unshared
@pytest.mark.parametrize("cfg", ["tiny", "gqa_small"])
def test_shared_slots_equal_private_recompute(cfg):
    """Run the request script through the tree, place every computed token's K/V at
    its slot, then attend through each request's slot list: the result must equal
    attention over the request's own private K/V, exactly, because every reused slot
    holds exactly the content of the position it is reused for."""
    if cfg == "tiny":
        w = config(1)
    else:
        w = few_shot(21, gqa128_shape(), 70, 6, 19, 5, name="gqa_small", q_rows=512)
    log = run_episode(w)
    content = np.full(w.pool_slots, -1, np.int64)
    k_tab, v_tab, _ = w.kv_table()
    checked = 0
    for rnd in log.rounds:
        for b, a in enumerate(rnd.admissions):
            r = w.requests[a.rid]
            # reused slots hold this request's content
            assert np.array_equal(content[a.row[:a.prefix_len]], r.kv_ids[:a.prefix_len])
            content[a.row[a.prefix_len:]] = r.kv_ids[a.prefix_len:]
            dec = rnd.decode_slots[:, b]
            content[dec] = r.out_kv_ids[:len(dec)]
            full_row = np.concatenate([a.row, dec])
            k_pool = decode_storage(k_tab[w.kv_rows(np.maximum(content, 0))], w.shape.kv_dtype)
            v_pool = decode_storage(v_tab[w.kv_rows(np.maximum(content, 0))], w.shape.kv_dtype)
            pos = np.arange(a.prefix_len, a.prompt_len + len(dec))
            if len(pos) == 0:
                continue
            from oracle.attention import request_q
            q = request_q(w, a.rid, pos)
            o_pool, l_pool = attention_via_pool(q, k_pool, v_pool, full_row[:pos[-1] + 1], pos,
                                                w.shape.sm_scale)
            o_ref, l_ref = reference_outputs(w, a.rid, pos)
            np.testing.assert_array_equal(o_pool, o_ref)
            np.testing.assert_array_equal(l_pool, l_ref)
            checked += 1
    assert checked > 0


# ------------------------------------------------------------- storage decoding
def test_e4m3fn_decoding_matches_torch_for_every_byte():
    b = np.arange(256, dtype=np.uint8)
    mine = e4m3fn_to_float(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_bf16_decoding_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                 # finite patterns
    mine = bf16_bits_to_float(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_generator_rounding_matches_torch():
    """Input preparation: bf16 rounding and per-row fp8 quantisation behave as stated."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(5000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    rows = rng.standard_normal((16, 1, 576)).astype(np.float32)
    q8, sc = quantize_e4m3_rows(rows)
    back = decode_storage(q8, "fp8", sc)
    assert np.all(np.abs(back - rows) <= np.abs(rows) / 16 + sc[:, None, None] * 2.0 ** -9)
    assert np.allclose(np.abs(back).reshape(16, -1).max(axis=1), np.abs(rows).reshape(16, -1).max(axis=1),
                       rtol=1e-6)


def test_request_kv_mla_values_are_key_prefix():
    from workloads import mla_groups
    w = mla_groups(9, "fp8", 2, 8, 2, 4, 2, q_rows=64)
    k, v = request_kv(w, w.full_kv_ids(w.phases[1].rids[0]))
    np.testing.assert_array_equal(v, k[:, :, :512])


def test_request_kv_gqa_fp8_shares_the_token_scale():
    """GQA fp8: a token's K and V rows (all KV heads) are quantised with one scale,
    amax over both / 448, and the oracle decodes both with it: the decoded values sit
    within E4M3's rounding of the unquantised N(0,1) table values, and the largest
    magnitude over a token's K and V is reproduced exactly."""
    from workloads import _normal, few_shot, gqa128_shape
    w = few_shot(2, gqa128_shape("fp8"), 20, 2, 4, 1, q_rows=64)
    s = w.shape
    k_raw = _normal(np.random.default_rng([w.seed, 1]), (w.table_rows, s.num_kv_heads, s.head_dim_qk))
    v_raw = _normal(np.random.default_rng([w.seed, 2]), (w.table_rows, s.num_kv_heads, s.head_dim_v))
    ids = w.full_kv_ids(w.phases[1].rids[0])
    k, v = request_kv(w, ids)
    rows = w.kv_rows(ids)
    kr, vr = k_raw[rows].astype(np.float64), v_raw[rows].astype(np.float64)
    amax = np.maximum(np.abs(kr).reshape(len(rows), -1).max(1), np.abs(vr).reshape(len(rows), -1).max(1))
    sc = (amax / 448.0)[:, None, None]
    assert np.all(np.abs(k - kr) <= np.abs(kr) / 16 + sc * 2.0 ** -9 + 1e-12)
    assert np.all(np.abs(v - vr) <= np.abs(vr) / 16 + sc * 2.0 ** -9 + 1e-12)
    both = np.maximum(np.abs(k).reshape(len(rows), -1).max(1), np.abs(v).reshape(len(rows), -1).max(1))
    np.testing.assert_allclose(both, amax, rtol=1e-6)
