"""Pins of the oracle's attention core and KV-cache share (CPU, no GPU).

The pages state no attention formula; the reading taken (scaled dot-product
softmax, causal, the grouped-query head mapping) is pinned against torch's
fp64 scaled_dot_product_attention, closed forms (uniform keys, one
position), invariants (shifting every key by one vector, concatenating the
ranks' heads, decode equal to the last rows of a full causal pass) and the
pages' KV bytes per token.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import seeded_inputs as si

HEADS = (8, 2, 16)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sizes.json")


def qkv_plan(t, r, heads=HEADS, K=32):
    n_q, n_kv, d = heads
    return oracle.plan("qkv_col", K, (n_q + 2 * n_kv) * d, t, r, heads=heads)


def counts(p):
    n_q, n_kv, d = p["heads"]
    return p["q_heads"][1] - p["q_heads"][0], p["kv_heads"][1] - p["kv_heads"][0], d


def draw(fn, seed, shape, *args):
    """A seeded 2-D draw of the same element count, reshaped."""
    return fn(seed, (int(np.prod(shape[:-1])), shape[-1]), *args).reshape(shape)


def case(p, S, q_len, kv_len, seed, L_max=16, sigma=1.0):
    """Random QKV rows, caches with random earlier positions, new tokens appended."""
    QKV = si.normal_bf16(seed, (S * q_len, p["shard_n"]), sigma)
    Kc, Vc = oracle.kv_cache_new(p, S + 1, L_max)
    Kc[:] = draw(si.normal_bf16, seed + 1, Kc.shape, sigma)
    Vc[:] = draw(si.normal_bf16, seed + 2, Vc.shape, sigma)
    slot = [(3 * s + 1) % (S + 1) for s in range(S)]
    oracle.kv_append(QKV, p, q_len, kv_len, slot, Kc, Vc)
    return QKV, Kc, Vc, slot


@pytest.mark.parametrize("t,r", [(1, 0), (2, 1), (4, 3), (8, 5)])
def test_square_causal_matches_torch_sdpa(t, r):
    """One sequence whose new tokens are its whole cache: torch's fp64 SDPA
    with is_causal and its own grouped-query mapping (query head h reads
    key-value head h // (heads / kv heads)) on the rank's heads."""
    p = qkv_plan(t, r)
    nq, nkv, d = counts(p)
    L = 7
    QKV, Kc, Vc, slot = case(p, 1, L, [L], 10 + t)
    got = oracle.attention_f64(QKV, p, L, [L], slot, Kc, Vc)
    q = torch.from_numpy(oracle.bf16_to_f64(QKV[:, :nq * d]).reshape(L, nq, d).transpose(1, 0, 2))[None]
    k = torch.from_numpy(oracle.bf16_to_f64(Kc[slot[0], :, :L]))[None]
    v = torch.from_numpy(oracle.bf16_to_f64(Vc[slot[0], :, :L]))[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)[0]
    ref = ref.numpy().transpose(1, 0, 2).reshape(L, nq * d)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_new_tokens_are_the_last_rows_of_a_full_pass():
    """Three new tokens on a cache of six equal rows 6..8 of a causal pass
    over all nine: new token i sits at position kv_len - q_len + i."""
    p = qkv_plan(2, 0)
    QKV = si.normal_bf16(20, (9, p["shard_n"]), 1.0)
    Kf, Vf = oracle.kv_cache_new(p, 1, 9)
    oracle.kv_append(QKV, p, 9, [9], [0], Kf, Vf)
    full = oracle.attention_f64(QKV, p, 9, [9], [0], Kf, Vf)
    Kc, Vc = oracle.kv_cache_new(p, 1, 9)
    oracle.kv_append(QKV[:6], p, 6, [6], [0], Kc, Vc)
    oracle.kv_append(QKV[6:], p, 3, [9], [0], Kc, Vc)
    np.testing.assert_array_equal(Kc, Kf)
    np.testing.assert_array_equal(oracle.attention_f64(QKV[6:], p, 3, [9], [0], Kc, Vc), full[6:])


def test_uniform_keys_average_the_visible_values():
    """Equal keys give equal weights: each query's output is the mean of the
    values at positions 0..p."""
    p = qkv_plan(1, 0)
    nq, nkv, d = counts(p)
    QKV, Kc, Vc, slot = case(p, 2, 3, [5, 8], 30)
    Kc[:] = Kc[:, :, :1, :]
    got = oracle.attention_f64(QKV, p, 3, [5, 8], slot, Kc, Vc)
    group = nq // nkv
    for row in range(6):
        s, i = divmod(row, 3)
        pos = [5, 8][s] - 3 + i
        for h in range(nq):
            want = oracle.bf16_to_f64(Vc[slot[s], h // group, :pos + 1]).mean(axis=0)
            np.testing.assert_allclose(got[row, h * d:(h + 1) * d], want, rtol=0, atol=1e-13)


def test_one_position_returns_its_value_exactly():
    p = qkv_plan(2, 1)
    nq, nkv, d = counts(p)
    QKV, Kc, Vc, slot = case(p, 3, 1, [1, 1, 1], 40)
    got = oracle.attention(QKV, p, 1, [1, 1, 1], slot, Kc, Vc)
    for s in range(3):
        for h in range(nq):
            np.testing.assert_array_equal(got[s, h * d:(h + 1) * d], Vc[slot[s], h // (nq // nkv), 0])


def test_shifting_every_key_changes_nothing():
    """q . (k + c) = q . k + q . c: the same shift for every position leaves
    the softmax unchanged. Integer keys and shift keep the bf16 sums exact."""
    p = qkv_plan(1, 0)
    QKV = si.int_bf16(50, (4, p["shard_n"]), -2, 2)
    Kc, Vc = oracle.kv_cache_new(p, 1, 8)
    Kc[:] = draw(si.int_bf16, 51, Kc.shape, -3, 3)
    Vc[:] = draw(si.normal_bf16, 52, Vc.shape, 1.0)
    oracle.kv_append(QKV, p, 4, [8], [0], Kc, Vc)
    base = oracle.attention_f64(QKV, p, 4, [8], [0], Kc, Vc)
    c = oracle.bf16_to_f64(draw(si.int_bf16, 53, (Kc.shape[1], 1, Kc.shape[3]), -4, 4))
    Ks = oracle.round_bf16(oracle.bf16_to_f64(Kc) + c)
    np.testing.assert_array_equal(oracle.bf16_to_f64(Ks), oracle.bf16_to_f64(Kc) + c)  # exact
    np.testing.assert_allclose(oracle.attention_f64(QKV, p, 4, [8], [0], Ks, Vc), base, rtol=0, atol=1e-12)


@pytest.mark.parametrize("t", [2, 4, 8])
def test_ranks_heads_concatenate_to_the_unsharded_attention(t):
    """X W_qkv cut per rank, each rank's cache and attention on its heads: the
    ranks' outputs side by side are the unsharded layer's, bit for bit."""
    n_q, n_kv, d = HEADS
    K, N = 32, (n_q + 2 * n_kv) * d
    X = si.normal_bf16(60, (6, K), 1.0)
    W = si.normal_bf16(61, (K, N), 0.2)
    p1 = qkv_plan(1, 0)
    QKV1 = oracle.col_linear_bf16(X, W, p1)
    K1, V1 = oracle.kv_cache_new(p1, 1, 6)
    oracle.kv_append(QKV1, p1, 6, [6], [0], K1, V1)
    whole = oracle.attention(QKV1, p1, 6, [6], [0], K1, V1)
    parts = []
    for r in range(t):
        p = qkv_plan(t, r)
        QKV = oracle.col_linear_bf16(X, W, p)
        Kc, Vc = oracle.kv_cache_new(p, 1, 6)
        oracle.kv_append(QKV, p, 6, [6], [0], Kc, Vc)
        parts.append(oracle.attention(QKV, p, 6, [6], [0], Kc, Vc))
        # the rank's cache holds exactly its key-value heads of the unsharded cache
        k0, k1 = p["kv_heads"]
        np.testing.assert_array_equal(Kc[0], K1[0, k0:k1])
        np.testing.assert_array_equal(Vc[0], V1[0, k0:k1])
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), whole)


def test_replicated_key_value_heads_hold_the_same_cache():
    """Past n_kv ranks, ranks r with the same floor(r n_kv / t) keep identical
    caches (the repeat the pages call wasted KV memory)."""
    n_q, n_kv, d = HEADS
    X = si.normal_bf16(70, (3, 32), 1.0)
    W = si.normal_bf16(71, (32, (n_q + 2 * n_kv) * d), 0.2)
    caches = {}
    for r in range(8):
        p = qkv_plan(8, r)
        assert p["kv_replicated"]
        Kc, Vc = oracle.kv_cache_new(p, 1, 3)
        oracle.kv_append(oracle.col_linear_bf16(X, W, p), p, 3, [3], [0], Kc, Vc)
        caches.setdefault(p["kv_heads"], []).append((Kc, Vc))
    assert sorted(caches) == [(0, 1), (1, 2)]
    for same in caches.values():
        assert len(same) == 4
        for Kc, Vc in same[1:]:
            np.testing.assert_array_equal(Kc, same[0][0])
            np.testing.assert_array_equal(Vc, same[0][1])


def test_kv_bytes_per_token_match_the_pages():
    g = json.load(open(GOLDEN))["kv_per_token"]
    n_q, n_kv, d = g["heads"]
    N = (n_q + 2 * n_kv) * d
    p1 = oracle.plan("qkv_col", 8192, N, 1, 0, heads=tuple(g["heads"]))
    assert oracle.kv_bytes_per_token(p1, g["layers"]) == g["bytes_t1"] == 320 * 1024
    for t, want in g["per_rank"]:
        for r in (0, t - 1):
            p = oracle.plan("qkv_col", 8192, N, t, r, heads=tuple(g["heads"]))
            assert oracle.kv_bytes_per_token(p, g["layers"]) == want


def test_planted_wrong_head_mapping_is_caught(monkeypatch):
    """A plausible mistake -- query head h reading key-value head h % n_kv
    instead of h // group -- must fail the library pin."""
    p = qkv_plan(1, 0)
    nq, nkv, d = counts(p)
    real = oracle._attn_heads

    def wrong(pp):
        a, b, c, _ = real(pp)
        return a, b, c, [h % b for h in range(a)]

    QKV, Kc, Vc, slot = case(p, 1, 5, [5], 80)
    monkeypatch.setattr(oracle, "_attn_heads", wrong)
    got = oracle.attention_f64(QKV, p, 5, [5], slot, Kc, Vc)
    q = torch.from_numpy(oracle.bf16_to_f64(QKV[:, :nq * d]).reshape(5, nq, d).transpose(1, 0, 2))[None]
    k = torch.from_numpy(oracle.bf16_to_f64(Kc[slot[0], :, :5]))[None]
    v = torch.from_numpy(oracle.bf16_to_f64(Vc[slot[0], :, :5]))[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)[0]
    ref = ref.numpy().transpose(1, 0, 2).reshape(5, nq * d)
    assert np.abs(got - ref).max() > 1e-3
