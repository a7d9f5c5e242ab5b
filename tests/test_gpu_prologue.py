"""GPU parity: fused QK-RMSNorm + partial RoPE + gate split + paged K/V write."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import bf16
from oracle import prologue as Pr
from gpu_util import DEV, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, lens, T, H_q, H_kv, D, R, P, base=10000.0, eps=1e-6):
    # only the pages that receive the T new tokens are mapped; the rest of
    # each page-table row is -1 (the prologue never reads those entries)
    n = len(lens)
    max_pages = max(-(-L // P) for L in lens) + 1
    needed = [sorted({p // P for p in range(L - T, L)}) for L in lens]
    N = sum(len(x) for x in needed) + 2
    perm = synth.permutation(N, synth.seed_of(seed, 0))
    pt = np.full((n, max_pages), -1, np.int32)
    at = 0
    for s, pages in enumerate(needed):
        for lp in pages:
            pt[s, lp] = perm[at]
            at += 1
    qg = synth.normal_bf16((n, T, H_q, 2, D), synth.seed_of(seed, 1))
    k = synth.normal_bf16((n, T, H_kv, D), synth.seed_of(seed, 2))
    v = synth.normal_bf16((n, T, H_kv, D), synth.seed_of(seed, 3))
    w_q = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 4))
    w_k = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 5))
    k_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 6))
    v_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 7))
    lens = np.asarray(lens, np.int32)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    print("case seed=%d lens=%s T=%d H_q=%d H_kv=%d D=%d R=%d P=%d" % (seed, list(lens), T, H_q, H_kv, D, R, P),
          flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q_out, gate = had.qk_norm_rope_gate(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt),
                                        to_dev(lens), kd, vd, R, base, eps, d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    return dict(qg=qg, k=k, v=v, w_q=w_q, w_k=w_k, pt=pt, lens=lens, k_pool=k_pool, v_pool=v_pool, kd=kd, vd=vd,
                q_out=q_out, gate=gate, P=P, T=T, R=R, base=base, eps=eps)


def _within_one_ulp(got_bits, ref):
    got = bf16.to_f64(got_bits)
    return np.all(np.abs(got - ref) <= bf16.ulp(ref))


@pytest.mark.parametrize("D,R,H_q,T", [(256, 64, 8, 1), (64, 16, 4, 1), (128, 128, 16, 4), (256, 64, 16, 4)])
def test_prologue_matches_oracle(D, R, H_q, T):
    c = _case(10 + D + T, [50001, 17, 1048576], T, H_q, 1, D, R, 64)
    kb, vb = bits_of(c["kd"]), bits_of(c["vd"])
    for s, L in enumerate(c["lens"]):
        pos = np.arange(L - T, L)
        q_ref, g_ref, k_ref, v_ref = Pr.qk_norm_rope_gate(
            bf16.to_f64(bits_of(c["qg"])[s]), bf16.to_f64(bits_of(c["k"])[s]), bf16.to_f64(bits_of(c["v"])[s]),
            c["w_q"].numpy().astype(np.float64), c["w_k"].numpy().astype(np.float64), pos, R, c["base"], c["eps"])
        assert _within_one_ulp(bits_of(c["q_out"])[s], q_ref)
        assert np.array_equal(bits_of(c["gate"])[s], bits_of(c["qg"])[s, :, :, 1])
        for j, p in enumerate(pos):
            page = c["pt"][s, p // c["P"]]
            assert _within_one_ulp(kb[page, :, p % c["P"]], k_ref[j])
            assert np.array_equal(vb[page, :, p % c["P"]], bits_of(c["v"])[s, j])


def test_prologue_touches_only_the_new_rows():
    c = _case(77, [130, 64], 2, 8, 2, 128, 32, 16)
    kb, vb = bits_of(c["kd"]), bits_of(c["vd"])
    mask = np.ones(kb.shape[:1] + kb.shape[2:3], bool)   # [page, row]
    for s, L in enumerate(c["lens"]):
        for p in range(L - 2, L):
            mask[c["pt"][s, p // 16], p % 16] = False
    for h in range(2):
        assert np.array_equal(kb[:, h][mask], bits_of(c["k_pool"])[:, h][mask])
        assert np.array_equal(vb[:, h][mask], bits_of(c["v_pool"])[:, h][mask])


def test_position_zero_is_plain_rmsnorm():
    c = _case(78, [1], 1, 4, 1, 64, 64, 16)
    q_ref = Pr.rmsnorm(bf16.to_f64(bits_of(c["qg"])[0, :, :, 0]), c["w_q"].numpy().astype(np.float64), c["eps"])
    assert _within_one_ulp(bits_of(c["q_out"])[0], q_ref)
