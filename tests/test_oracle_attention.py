"""Pins for the oracle's decode attention, split partials and merge (CPU)."""

import math

import numpy as np
import torch

from oracle import attention as A
from oracle import bf16, paging


def _brute(q, K, V, sm_scale):
    """Scalar triple loop: softmax over visible keys, causal inside the draft."""
    q_len, H_q, D = q.shape
    L, H_kv, Dv = V.shape
    G = H_q // H_kv
    out = np.zeros((q_len, H_q, Dv))
    for j in range(q_len):
        n = L - q_len + j + 1
        for hq in range(H_q):
            h = hq // G
            s = [sm_scale * sum(q[j, hq, d] * K[t, h, d] for d in range(D)) for t in range(n)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = sum(w)
            for d in range(Dv):
                out[j, hq, d] = sum(w[t] * V[t, h, d] for t in range(n)) / z
    return out


def test_matches_brute_force():
    rng = np.random.default_rng(0)
    for q_len, H_q, H_kv, D, L in [(1, 4, 1, 8, 9), (3, 4, 2, 5, 7), (2, 2, 2, 3, 2)]:
        q = rng.standard_normal((q_len, H_q, D))
        K = rng.standard_normal((L, H_kv, D))
        V = rng.standard_normal((L, H_kv, D))
        np.testing.assert_allclose(A.attention(q, K, V, 0.7), _brute(q, K, V, 0.7), atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    L, D = 50, 16
    K = np.repeat(rng.standard_normal((1, 1, D)), L, axis=0)
    V = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 4, D))
    o = A.attention(q, K, V, 1 / 4)
    np.testing.assert_allclose(o[0], np.repeat(V[:, 0].mean(0)[None], 4, 0), atol=1e-13)
    # the same with a scale of zero and arbitrary keys
    K2 = rng.standard_normal((L, 1, D))
    np.testing.assert_allclose(A.attention(q, K2, V, 0.0)[0, 2], V[:, 0].mean(0), atol=1e-13)


def test_one_token_context_returns_v():
    rng = np.random.default_rng(2)
    V = rng.standard_normal((1, 1, 8))
    o = A.attention(rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 1, 8)), V, 0.3)
    assert np.array_equal(o[0, 0], V[0, 0]) and np.array_equal(o[0, 1], V[0, 0])


def test_dominant_score_selects_its_value():
    rng = np.random.default_rng(3)
    L, D = 20, 8
    K = rng.standard_normal((L, 1, D)) * 0.01
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    K[7, 0, 0] = 1000.0
    V = rng.standard_normal((L, 1, D))
    np.testing.assert_allclose(A.attention(q, K, V, 1.0)[0, 0], V[7, 0], atol=1e-12)


def test_matches_torch_sdpa_fp64():
    # library special case: torch's scaled_dot_product_attention in float64
    rng = np.random.default_rng(4)
    q_len, H_q, H_kv, D, L = 4, 8, 2, 16, 37
    q = rng.standard_normal((q_len, H_q, D))
    K = rng.standard_normal((L, H_kv, D))
    V = rng.standard_normal((L, H_kv, D))
    G = H_q // H_kv
    mask = np.zeros((q_len, L), bool)
    for j in range(q_len):
        mask[j, : L - q_len + j + 1] = True
    tq = torch.from_numpy(q).permute(1, 0, 2)                          # [H_q, q_len, D]
    tk = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2)    # [H_q, L, D]
    tv = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.25).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(A.attention(q, K, V, 0.25), ref, atol=1e-12)


def test_paged_equals_contiguous():
    rng = np.random.default_rng(5)
    P, H_kv, D, H_q, q_len = 16, 1, 32, 4, 2
    L = 70
    Kb = bf16.from_f64(rng.standard_normal((L, H_kv, D)))
    Vb = bf16.from_f64(rng.standard_normal((L, H_kv, D)))
    qb = bf16.from_f64(rng.standard_normal((1, q_len, H_q, D)))
    pages = rng.permutation(12)[:5]
    kp = np.zeros((12, H_kv, P, D), np.uint16)
    vp = np.zeros((12, H_kv, P, D), np.uint16)
    paging.scatter_contiguous(Kb, pages, P, kp)
    paging.scatter_contiguous(Vb, pages, P, vp)
    pt = np.full((1, 6), -1, np.int32)
    pt[0, :5] = pages
    o = A.paged_attention(qb, kp, vp, pt, np.array([L]), P, 0.2)
    ref = A.attention(bf16.to_f64(qb[0]), bf16.to_f64(Kb), bf16.to_f64(Vb), 0.2)
    assert np.array_equal(o[0], ref)


def test_split_partials_merge_to_the_unsplit_result():
    rng = np.random.default_rng(6)
    q_len, H_q, H_kv, D, L = 4, 8, 1, 16, 100
    q = rng.standard_normal((q_len, H_q, D))
    K = rng.standard_normal((L, H_kv, D))
    V = rng.standard_normal((L, H_kv, D))
    ref = A.attention(q, K, V, 0.25)
    for bounds in ([(0, L)], [(0, 30), (30, 64), (64, 100)], [(0, 97), (97, 98), (98, 99), (99, 128), (128, 192)]):
        o, m, l = A.split_partials(q, K, V, 0.25, bounds)
        np.testing.assert_allclose(A.lse_merge(o, m, l), ref, atol=1e-12)
    # a split beyond every query's visible range is empty
    o, m, l = A.split_partials(q, K, V, 0.25, [(0, 100), (100, 164)])
    assert np.all(m[1] == -np.inf) and np.all(l[1] == 0) and np.all(o[1] == 0)
    # query j sees keys < 97 + j: the split [98, 100) is empty for j = 0, 1
    o, m, l = A.split_partials(q, K, V, 0.25, [(0, 98), (98, 100)])
    assert np.isneginf(m[1, :2]).all() and np.isfinite(m[1, 2:]).all()


def test_single_split_merge_is_identity():
    rng = np.random.default_rng(8)
    o = rng.standard_normal((1, 2, 3, 5))
    m = rng.standard_normal((1, 2, 3))
    l = rng.random((1, 2, 3)) + 0.5
    np.testing.assert_allclose(A.lse_merge(o, m, l), o[0] / l[0][..., None], rtol=1e-15)
