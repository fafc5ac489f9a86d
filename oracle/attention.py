"""Oracle: exact softmax attention per request, in fp64 (fp32 on request).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed is the plain definition. A request's query at absolute
position p attends to that request's own keys at positions 0..p (causal,
inclusive of itself), as if nothing were shared: the page "49 · RadixAttention,
eviction và cache churn" (§2) reuses the shared part and computes only the new
part, which must give the same numbers as recomputing everything. Prefill of
all new prompt tokens at once against the cached prefix is the extend phase;
one token per step is decode (AWS blog "Improve performance of Falcon models
with Amazon SageMaker", sections on the KV cache and on batching).

Per query head h (KV head h // (Hq/Hkv)):
    s_j = sm_scale * <q, k_j>,  w_j = exp(s_j - max s),
    o = sum_j w_j v_j / sum_j w_j,  lse = max s + log sum_j w_j.
MLA (SGLang feature article, §一): one latent KV head; the score uses all 576
dims of the row, the output reads its first 512 dims.

Storage decoding: bf16 is the upper half of an IEEE binary32; fp8 E4M3 (OCP
'fn': bias 7, no infinities, S.1111.111 = NaN, max 448) times the token's
fp32 scale (KV Cache FP8, SGLang feature article §一; one scale per token,
shared by the token's K and V rows of every KV head where V is stored apart).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_float(u16: np.ndarray, dtype=np.float64) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype)


def e4m3fn_to_float(u8: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Decode OCP E4M3FN bytes from the format definition."""
    b = np.asarray(u8, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7 == 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return (sign * val).astype(dtype)


def decode_storage(x: np.ndarray, kind: str, scale=None, dtype=np.float64) -> np.ndarray:
    """Turn stored K/V/Q values into floats: kind 'f32' | 'bf16' | 'fp8'."""
    if kind == "f32":
        return np.asarray(x, dtype=np.float32).astype(dtype)
    if kind == "bf16":
        return bf16_bits_to_float(x, dtype)
    if kind == "fp8":
        v = e4m3fn_to_float(x, dtype)
        s = np.asarray(scale, dtype=np.float32).astype(dtype)
        return v * s.reshape((-1,) + (1,) * (v.ndim - 1))
    raise ValueError(kind)


def attention(q, k, v, q_pos, sm_scale, dtype=np.float64):
    """Causal softmax attention for one request.

    q: [n, Hq, Dqk] queries at absolute positions q_pos [n];
    k: [L, Hkv, Dqk], v: [L, Hkv, Dv] the request's keys/values at positions 0..L-1.
    Returns (o [n, Hq, Dv], lse [n, Hq]) in ``dtype``.
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, hq, _ = q.shape
    L, hkv, _ = k.shape
    dv = v.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if n and (q_pos.max() >= L or q_pos.min() < 0):
        raise ValueError("query position outside the key range")
    group = hq // hkv
    scale = dtype(sm_scale)
    visible = np.arange(L)[None, :] <= q_pos[:, None]          # [n, L]
    o = np.zeros((n, hq, dv), dtype=dtype)
    lse = np.zeros((n, hq), dtype=dtype)
    for h in range(hq):
        kh = h // group
        s = (q[:, h, :] @ k[:, kh, :].T) * scale                # [n, L]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        den = w.sum(axis=1, keepdims=True)
        o[:, h, :] = (w @ v[:, kh, :]) / den
        lse[:, h] = m[:, 0] + np.log(den[:, 0])
    return o, lse


def request_kv(workload, kv_ids, dtype=np.float64):
    """Logical K/V of a request from its content ids: (K [L, Hkv, Dqk], V [L, Hkv, Dv])."""
    s = workload.shape
    k_tab, v_tab, k_scale = workload.kv_table()
    rows = workload.kv_rows(kv_ids)
    if s.kv_dtype == "fp8":
        k = decode_storage(k_tab[rows], "fp8", k_scale[rows], dtype)
    else:
        k = decode_storage(k_tab[rows], s.kv_dtype, None, dtype)
    if s.v_is_k_prefix:
        v = k[:, :, :s.head_dim_v]
    elif s.kv_dtype == "fp8":   # the token's one scale serves its K and V rows
        v = decode_storage(v_tab[rows], "fp8", k_scale[rows], dtype)
    else:
        v = decode_storage(v_tab[rows], s.kv_dtype, None, dtype)
    return k, v


def request_q(workload, rid, positions, dtype=np.float64):
    qt = workload.q_table()
    return decode_storage(qt[workload.q_index(rid, positions)], workload.shape.q_dtype, None, dtype)


def reference_outputs(workload, rid, positions, dtype=np.float64):
    """Oracle output of request ``rid`` for queries at ``positions`` (extend or decode):
    keys are the request's own tokens 0..max(positions)."""
    positions = np.asarray(positions, dtype=np.int64)
    L = int(positions.max()) + 1
    ids = workload.full_kv_ids(rid)[:L]
    k, v = request_kv(workload, ids, dtype)
    q = request_q(workload, rid, positions, dtype)
    return attention(q, k, v, positions, workload.shape.sm_scale, dtype)


def attention_via_pool(q, k_pool, v_pool, row_slots, q_pos, sm_scale, dtype=np.float64):
    """Same attention, keys gathered from a slot pool through the request's slot list."""
    row = np.asarray(row_slots, dtype=np.int64)
    return attention(q, k_pool[row], v_pool[row], q_pos, sm_scale, dtype)
