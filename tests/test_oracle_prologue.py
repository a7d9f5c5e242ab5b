"""Pins for the oracle's RMSNorm + partial RoPE + gate split (CPU)."""

import numpy as np
import torch

from oracle import prologue as Pr


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 4, 64))
    w = rng.random(64) + 0.5
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(Pr.rmsnorm(x, w, 1e-6), ref, rtol=1e-13)


def test_rmsnorm_hand_example_and_unit_rms():
    # x = [3, 4, 0, 0]: mean square 25/4, rms 2.5 -> [1.2, 1.6, 0, 0]
    y = Pr.rmsnorm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.ones(4), 0.0)
    np.testing.assert_allclose(y, [[1.2, 1.6, 0.0, 0.0]], rtol=1e-15)
    rng = np.random.default_rng(1)
    z = Pr.rmsnorm(rng.standard_normal((5, 256)), np.ones(256), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(z * z, axis=-1)), 1.0, rtol=1e-14)


def test_rope_position_zero_is_identity_and_tail_untouched():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((3, 2, 32))
    np.testing.assert_array_equal(Pr.rope_partial(y, [0, 0, 0], 16, 10000.0), y)
    r = Pr.rope_partial(y, [5, 900, 123456], 16, 10000.0)
    np.testing.assert_array_equal(r[..., 16:], y[..., 16:])


def test_rope_matches_complex_rotation():
    # rotate-half pairing as complex numbers: z_i = y_i + 1j*y_{i+R/2}, times exp(1j*theta_i)
    rng = np.random.default_rng(3)
    R, D = 64, 256
    y = rng.standard_normal((4, 3, D))
    pos = np.array([1, 17, 50000, 1048575])
    z = y[..., : R // 2] + 1j * y[..., R // 2:R]
    theta = pos[:, None, None] * 10000.0 ** (-(np.arange(R // 2) * 2.0) / R)
    zr = z * np.exp(1j * theta)
    got = Pr.rope_partial(y, pos, R, 10000.0)
    np.testing.assert_allclose(got[..., : R // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(got[..., R // 2:R], zr.imag, atol=1e-12)


def test_rope_preserves_pair_norms_and_is_relative():
    rng = np.random.default_rng(4)
    R = 16
    a = rng.standard_normal((1, 1, R))
    b = rng.standard_normal((1, 1, R))
    ra = Pr.rope_partial(a, [7], R, 10000.0)
    np.testing.assert_allclose(ra[..., :8] ** 2 + ra[..., 8:] ** 2, a[..., :8] ** 2 + a[..., 8:] ** 2, rtol=1e-12)
    dots = []
    for m in (3, 40, 1000):
        x = Pr.rope_partial(a, [m + 5], R, 10000.0)
        z = Pr.rope_partial(b, [m], R, 10000.0)
        dots.append(float(np.sum(x * z)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-11)


def test_fused_prologue_composition():
    rng = np.random.default_rng(5)
    T, Hq, Hkv, D, R = 2, 4, 1, 32, 8
    qg = rng.standard_normal((T, Hq, 2, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    wq = rng.random(D) + 0.5
    wk = rng.random(D) + 0.5
    pos = np.array([100, 101])
    q_out, gate, k_out, v_out = Pr.qk_norm_rope_gate(qg, k, v, wq, wk, pos, R, 10000.0, 1e-6)
    np.testing.assert_array_equal(gate, qg[:, :, 1])
    np.testing.assert_array_equal(v_out, v)
    # norm then rotate: rotation keeps the per-pair norms of the normed vector
    qn = Pr.rmsnorm(qg[:, :, 0], wq, 1e-6)
    np.testing.assert_allclose(q_out[..., R:], qn[..., R:], rtol=1e-15)
    np.testing.assert_allclose(np.hypot(q_out[..., :4], q_out[..., 4:8]), np.hypot(qn[..., :4], qn[..., 4:8]), rtol=1e-12)
    kn = Pr.rmsnorm(k, wk, 1e-6)
    np.testing.assert_allclose(k_out, Pr.rope_partial(kn, pos, R, 10000.0), rtol=1e-15)


def test_rope_frequencies_at_known_angles():
    # pair 0 turns by exactly pos radians; pair R/4 turns by pos / sqrt(base)
    R, D = 64, 256
    y = np.zeros((2, 1, D))
    y[0, 0, 0] = 1.0
    y[1, 0, 16] = 1.0
    r = Pr.rope_partial(y, [1, 100], R, 10000.0)
    np.testing.assert_allclose([r[0, 0, 0], r[0, 0, 32]], [np.cos(1.0), np.sin(1.0)], atol=1e-15)
    np.testing.assert_allclose([r[1, 0, 16], r[1, 0, 48]], [np.cos(1.0), np.sin(1.0)], atol=1e-14)
    assert np.count_nonzero(r[0]) == 2 and np.count_nonzero(r[1]) == 2


def test_output_gate_special_values_and_symmetry():
    rng = np.random.default_rng(9)
    o = rng.standard_normal((3, 4, 32))
    g = rng.standard_normal((3, 4, 32)) * 4
    # sigmoid(0) = 1/2 exactly; sigmoid(x) + sigmoid(-x) = 1
    np.testing.assert_array_equal(Pr.output_gate(o, np.zeros_like(o)), o / 2)
    np.testing.assert_allclose(Pr.output_gate(o, g) + Pr.output_gate(o, -g), o, rtol=1e-14, atol=1e-15)
    # saturation: a large gate passes the output, a very negative one closes it
    np.testing.assert_allclose(Pr.output_gate(o, np.full_like(o, 60.0)), o, rtol=1e-15)
    assert np.max(np.abs(Pr.output_gate(o, np.full_like(o, -60.0)))) < 1e-25
    # agrees with the library's logistic function
    from scipy.special import expit
    np.testing.assert_allclose(Pr.output_gate(o, g), o * expit(g), rtol=1e-14)
    # the gate acts per element, not per head (a swapped axis would fail)
    g2 = g.copy()
    g2[..., 0] = 30.0
    assert np.allclose(Pr.output_gate(o, g2)[..., 0], o[..., 0])
    assert np.allclose(Pr.output_gate(o, g2)[..., 1:], Pr.output_gate(o, g)[..., 1:])
