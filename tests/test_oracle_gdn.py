"""Pins for the oracle's gated delta rule (CPU)."""

import os

import numpy as np
import pytest

from oracle import gdn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "gdn_step_2x2.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                vals.setdefault(line.split()[0], []).append(line.split()[1:])
    return vals


def test_hand_worked_2x2():
    g = _golden()
    f = lambda xs: np.array([float(x) for x in xs])
    S0 = f(g["S0"][0]).reshape(2, 2)
    t1 = g["token1"][0]
    k, v, a, b = f(t1[1:3]), f(t1[4:6]), float(t1[7]), float(t1[9])
    for row in g["o1"]:
        q = f(row[1:3])
        S1, o = gdn.step(S0, q, k, v, a, b)
        np.testing.assert_allclose(S1, f(g["S1"][0]).reshape(2, 2), rtol=0, atol=1e-15)
        np.testing.assert_allclose(o, f(row[4:6]), atol=1e-15)
    t2 = g["token2"][0]
    S2, _ = gdn.step(S1, np.zeros(2), f(t2[1:3]), f(t2[4:6]), float(t2[7]), float(t2[9]))
    np.testing.assert_allclose(S2, f(g["S2"][0]).reshape(2, 2), atol=1e-14)


def test_scalar_loop_definition():
    # entrywise: S'[i,j] = a * sum_m S[i,m] (delta_mj - b k_m k_j) + b v_i k_j
    rng = np.random.default_rng(0)
    dv, dk = 3, 4
    S = rng.standard_normal((dv, dk))
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    a, b = 0.93, 0.41
    ref = np.zeros((dv, dk))
    for i in range(dv):
        for j in range(dk):
            acc = 0.0
            for m in range(dk):
                acc += S[i, m] * ((1.0 if m == j else 0.0) - b * k[m] * k[j])
            ref[i, j] = a * acc + b * v[i] * k[j]
    S1, o = gdn.step(S, q, k, v, a, b)
    np.testing.assert_allclose(S1, ref, atol=1e-14)
    np.testing.assert_allclose(o, [sum(ref[i, j] * q[j] for j in range(dk)) for i in range(dv)], atol=1e-14)


def test_beta_zero_alpha_one_leaves_state_unchanged():
    rng = np.random.default_rng(1)
    S = rng.standard_normal((8, 8))
    T = 5
    states, _ = gdn.sequential(S, rng.standard_normal((T, 8)), _unit(rng, T, 8), rng.standard_normal((T, 8)),
                               np.ones(T), np.zeros(T))
    assert np.array_equal(states[-1], S)


def test_beta_zero_decays_by_product_of_alphas():
    rng = np.random.default_rng(2)
    S = rng.standard_normal((6, 6))
    al = rng.uniform(0.9, 1.0, 7)
    states, _ = gdn.sequential(S, rng.standard_normal((7, 6)), _unit(rng, 7, 6), rng.standard_normal((7, 6)),
                               al, np.zeros(7))
    np.testing.assert_allclose(states[-1], np.prod(al) * S, rtol=1e-13)


def test_retrieval_identity():
    rng = np.random.default_rng(3)
    d = 16
    S = rng.standard_normal((d, d))
    for _ in range(5):
        k = rng.standard_normal(d)
        v = rng.standard_normal(d)
        a, b = rng.uniform(0.9, 1), rng.uniform(0, 1)
        S1, _ = gdn.step(S, k, k, v, a, b)
        kk = k @ k
        np.testing.assert_allclose(S1 @ k, a * (1 - b * kk) * (S @ k) + b * kk * v, atol=1e-10)
        # unit key and beta = 1: writing (k, v) then querying with k returns v
        ku = k / np.linalg.norm(k)
        S2, o = gdn.step(S, ku, ku, v, a, 1.0)
        np.testing.assert_allclose(o, v, atol=1e-12)
        # the transposed orientation does not have this property
        assert np.max(np.abs(S2.T @ ku - v)) > 1e-3
        S = S1


def test_chunked_equals_sequential():
    rng = np.random.default_rng(4)
    T, dk, dv = 37, 8, 6
    S0 = rng.standard_normal((dv, dk))
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    al, be = rng.uniform(0.9, 1.0, T), rng.uniform(0, 1, T)
    states, outs = gdn.sequential(S0, q, k, v, al, be, 0.5)
    for C in (1, 4, 16, 64):
        Sf, oc = gdn.chunked(S0, q, k, v, al, be, C, 0.5)
        np.testing.assert_allclose(Sf, states[-1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(oc, outs, rtol=1e-12, atol=1e-12)


def test_state_update_slots_and_checkpoints():
    rng = np.random.default_rng(5)
    n_slots, H, dv, dk, S_n, T = 8, 2, 4, 4, 2, 3
    pool = rng.standard_normal((n_slots, H, dv, dk)).astype(np.float32)
    in_idx = np.array([5, -1])
    out_idx = np.array([[1, 2, 3], [4, 6, 7]])
    q = rng.standard_normal((S_n, T, H, dk))
    k = rng.standard_normal((S_n, T, H, dk))
    v = rng.standard_normal((S_n, T, H, dv))
    al = rng.uniform(0.9, 1, (S_n, T, H))
    be = rng.uniform(0, 1, (S_n, T, H))
    new, o = gdn.state_update(pool, in_idx, out_idx, q, k, v, al, be)
    # untouched slots keep their bytes, including the shared input slot
    for sl in (0, 5):
        assert np.array_equal(new[sl], pool[sl])
    for h in range(H):
        st, outs = gdn.sequential(pool[5, h].astype(np.float64), q[0, :, h], k[0, :, h], v[0, :, h], al[0, :, h], be[0, :, h])
        for t in range(T):
            assert np.array_equal(new[out_idx[0, t], h], st[t].astype(np.float32))
        np.testing.assert_allclose(o[0, :, h], outs, rtol=1e-15)
        st0, _ = gdn.sequential(np.zeros((dv, dk)), q[1, :, h], k[1, :, h], v[1, :, h], al[1, :, h], be[1, :, h])
        assert np.array_equal(new[out_idx[1, -1], h], st0[-1].astype(np.float32))
    # in == out for a single token reads before it writes
    new2, _ = gdn.state_update(pool, np.array([3]), np.array([[3]]), q[:1, :1], k[:1, :1], v[:1, :1], al[:1, :1], be[:1, :1])
    st, _ = gdn.sequential(pool[3, 0].astype(np.float64), q[0, :1, 0], k[0, :1, 0], v[0, :1, 0], al[0, :1, 0], be[0, :1, 0])
    assert np.array_equal(new2[3, 0], st[0].astype(np.float32))


def test_rank_one_heads_match_dense_definition():
    # several heads, ragged magnitudes, q_scale != 1: the rank-one form used
    # for long chains equals the dense per-head recurrence
    rng = np.random.default_rng(7)
    H, T, dv, dk = 3, 9, 5, 6
    S0 = rng.standard_normal((H, dv, dk))
    q, k = rng.standard_normal((T, H, dk)), _unit(rng, T * H, dk).reshape(T, H, dk) * 1.3
    v = rng.standard_normal((T, H, dv))
    al, be = rng.uniform(0.8, 1.0, (T, H)), rng.uniform(0.0, 1.0, (T, H))
    S, o = gdn.sequential_heads(S0, q, k, v, al, be, q_scale=0.7)
    for h in range(H):
        st, oh = gdn.sequential(S0[h], q[:, h], k[:, h], v[:, h], al[:, h], be[:, h], q_scale=0.7)
        np.testing.assert_allclose(S[h], st[-1], atol=1e-12)
        np.testing.assert_allclose(o[:, h], oh, atol=1e-12)


def test_rank_one_heads_reproduce_hand_worked_2x2():
    g = _golden()
    f = lambda xs: np.array([float(x) for x in xs])
    S0 = f(g["S0"][0]).reshape(1, 2, 2)
    t1, t2 = g["token1"][0], g["token2"][0]
    k = np.stack([f(t1[1:3]), f(t2[1:3])])[:, None, :]
    v = np.stack([f(t1[4:6]), f(t2[4:6])])[:, None, :]
    al = np.array([[float(t1[7])], [float(t2[7])]])
    be = np.array([[float(t1[9])], [float(t2[9])]])
    S, _ = gdn.sequential_heads(S0, np.zeros((2, 1, 2)), k, v, al, be)
    np.testing.assert_allclose(S[0], f(g["S2"][0]).reshape(2, 2), atol=1e-14)


def test_raw_gates_parameterisation():
    from scipy.special import expit
    rng = np.random.default_rng(21)
    g = -np.abs(rng.standard_normal(50)) * 3
    b = rng.standard_normal(50) * 4
    al, be = gdn.gates_from_raw(g, b)
    np.testing.assert_allclose(al, np.exp(g), rtol=1e-15)
    np.testing.assert_allclose(be, expit(b), rtol=1e-14)
    assert np.all((al > 0) & (al <= 1)) and np.all((be > 0) & (be < 1))
    a0, b0 = gdn.gates_from_raw(0.0, 0.0)
    assert a0 == 1.0 and b0 == 0.5
    # a strongly negative b closes the write: the state decays by exp(sum g)
    rng = np.random.default_rng(22)
    S = rng.standard_normal((6, 6))
    T = 5
    gg = -rng.uniform(0, 0.2, T)
    al, be = gdn.gates_from_raw(gg, np.full(T, -800.0))
    assert np.all(be == 0.0)
    states, _ = gdn.sequential(S, rng.standard_normal((T, 6)), _unit(rng, T, 6), rng.standard_normal((T, 6)), al, be)
    np.testing.assert_allclose(states[-1], np.exp(gg.sum()) * S, rtol=1e-13)


def _prefill_case(rng, lens, H, dk, dv, n_slots):
    N = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = _unit(rng, N * H, dk).reshape(N, H, dk)
    k = _unit(rng, N * H, dk).reshape(N, H, dk)
    v = rng.standard_normal((N, H, dv))
    al = rng.uniform(0.85, 1.0, (N, H))
    be = rng.uniform(0.0, 1.0, (N, H))
    pool = rng.standard_normal((n_slots, H, dv, dk)).astype(np.float32)
    return cu, q, k, v, al, be, pool


def test_prefill_equals_the_chunked_form():
    # an independently derived evaluation (WY/UT chunks, ragged last chunk)
    rng = np.random.default_rng(31)
    lens, H, dk, dv = [37, 0, 70, 5], 2, 8, 6
    cu, q, k, v, al, be, pool = _prefill_case(rng, lens, H, dk, dv, 9)
    in_idx, out_idx = np.array([3, 4, -1, 3]), np.array([0, 5, 4, 8])
    new, o = gdn.prefill(pool, in_idx, out_idx, cu, q, k, v, al, be, q_scale=0.5)
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(H):
            S0 = np.zeros((dv, dk)) if in_idx[s] < 0 else pool[in_idx[s], h].astype(np.float64)
            for C in (1, 16, 64):
                S, oc = gdn.chunked(S0, q[a:b, h], k[a:b, h], v[a:b, h], al[a:b, h], be[a:b, h], C, q_scale=0.5)
                np.testing.assert_allclose(o[a:b, h], oc, atol=1e-11)
                np.testing.assert_allclose(new[out_idx[s], h], S.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_prefill_slot_semantics_and_closed_forms():
    rng = np.random.default_rng(32)
    lens, H, dk, dv = [0, 12, 9], 2, 4, 4
    cu, q, k, v, al, be, pool = _prefill_case(rng, lens, H, dk, dv, 6)
    be[cu[2]:cu[3]] = 0.0                                   # third sequence: no write, decay only
    in_idx, out_idx = np.array([1, 2, 2]), np.array([3, 2, 5])  # second sequence updates its slot in place
    new, o = gdn.prefill(pool, in_idx, out_idx, cu, q, k, v, al, be)
    # an empty sequence copies its input state
    assert np.array_equal(new[3], pool[1])
    # beta = 0: S = prod(alpha) S0, o_t = gamma_t S0 q_t; the input is slot 2 as it was before the call
    gam = np.cumprod(al[cu[2]:cu[3]], axis=0)
    for h in range(H):
        S0 = pool[2, h].astype(np.float64)
        np.testing.assert_allclose(new[5, h], (gam[-1, h] * S0).astype(np.float32), rtol=1e-6)
        np.testing.assert_allclose(o[cu[2]:cu[3], h], gam[:, h:h + 1] * (q[cu[2]:cu[3], h] @ S0.T), atol=1e-12)
    # untouched slots keep their bytes
    for sl in (0, 1, 4):
        assert np.array_equal(new[sl], pool[sl])
    assert not np.array_equal(new[2], pool[2])
