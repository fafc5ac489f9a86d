"""The seeded generators: content ids must follow token paths (a causal model's K/V
of a position depends only on the tokens up to it), shapes must match the stated
configurations, and generation must be deterministic."""
import numpy as np
import pytest

from workloads import agent_branch, chat_tree, config, cyclic_stream, few_shot, gqa128_shape, mla_groups, tiny_shape


def _check_content_ids(w):
    by_key, by_id = {}, {}
    for rid in range(len(w.requests)):
        toks, ids = w.full_tokens(rid), w.full_kv_ids(rid)
        parent = -1
        for t, i in zip(toks.tolist(), ids.tolist()):
            key = (parent, t)
            assert by_key.setdefault(key, i) == i, "same token path, different content"
            assert by_id.setdefault(i, key) == key, "same content, different token path"
            parent = i


@pytest.mark.parametrize("make", [
    lambda: config(1),
    lambda: few_shot(2, gqa128_shape(), 100, 40, 9, 3),
    lambda: chat_tree(3, tiny_shape(), 10, 4, 5, 20),
    lambda: agent_branch(4, tiny_shape(), 3, 50, 4, 20, 3, 5),
    lambda: cyclic_stream(4, tiny_shape(), 5, 30, 2, 4),
    lambda: mla_groups(5, "bf16", 3, 40, 5, 20, 4, q_rows=64),
])
def test_content_ids_follow_token_paths(make):
    _check_content_ids(make())


def test_config_shapes():
    w = config(2)
    assert len(w.phases[1].rids) == 256 and w.phases[1].n_decode == 128
    assert all(len(w.requests[r].tokens) == 2048 + 128 for r in w.phases[1].rids)
    s = w.shape
    assert (s.num_q_heads, s.num_kv_heads, s.head_dim_qk, s.q_dtype) == (32, 8, 128, "bf16")
    w4 = config(4)
    assert [len(p.rids) for p in w4.phases] == [16, 128, 512] and w4.phases[2].n_decode == 256
    w5 = config(5, "fp8")
    assert w5.shape.kv_dtype == "fp8" and w5.shape.head_dim_qk == 576 and w5.shape.num_kv_heads == 1
    assert len(w5.phases[1].rids) == 256
    assert all(len(w5.requests[r].tokens) == 4096 for r in w5.phases[1].rids)


def test_generation_is_deterministic():
    a, b = config(1), config(1)
    for ra, rb in zip(a.requests, b.requests):
        assert np.array_equal(ra.tokens, rb.tokens) and np.array_equal(ra.out_tokens, rb.out_tokens)
    assert np.array_equal(a.kv_table()[0], b.kv_table()[0])
    assert np.array_equal(a.q_table(), b.q_table())
