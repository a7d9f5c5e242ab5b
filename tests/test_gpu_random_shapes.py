"""GPU parity over seeded random shapes: decode attention (both paths,
gated or not, forced or planned splits), the fused layer, and the GDN
prefill (one pass and in 3-8 segments), each against the fp64 oracle.
The shapes are drawn once from a fixed seed, so every run checks the same
cases."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import attention as A
from oracle import bf16, gdn
from oracle import paging as PG
from oracle import prologue as Pr
from gpu_util import DEV, assert_attn_close, bits_of, paged_case, to_dev

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)


def _attn_cases(n):
    out = []
    while len(out) < n:
        G = int(_rng.choice([1, 2, 4, 8, 16, 32]))
        q_len = int(_rng.integers(1, 9))
        H_kv = int(_rng.integers(1, 3))
        if G * q_len > 256:
            continue
        D = int(_rng.choice([64, 128, 256]))
        P = int(_rng.choice([16, 32, 64]))
        lens = [int(x) for x in _rng.integers(q_len, 3000, int(_rng.integers(1, 4)))]
        splits = int(_rng.choice([0, 0, 1, 5, 37]))
        out.append((len(out), G, q_len, H_kv, D, P, lens, splits, bool(_rng.integers(0, 2)), bool(_rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _attn_cases(24), ids=lambda c: "attn%d" % c[0])
def test_random_attention_shapes(case):
    i, G, q_len, H_kv, D, P, lens, splits, det, gated = case
    seed = 8000 + i
    q, kp, vp, pt, L = paged_case(seed, lens, q_len, G * H_kv, H_kv, D, P)
    gate = synth.normal_bf16(tuple(q.shape), synth.seed_of(seed, 99)) if gated else None
    print("case %d: G=%d q_len=%d H_kv=%d D=%d P=%d lens=%s splits=%d det=%d gated=%d" % (
        i, G, q_len, H_kv, D, P, lens, splits, det, gated), flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = had.decode_attn(to_dev(q), to_dev(kp), to_dev(vp), to_dev(pt), to_dev(L), num_splits=splits, d_err=err,
                          deterministic=det, gate=None if gate is None else to_dev(gate))
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = A.paged_attention(bits_of(q), bits_of(kp), bits_of(vp), pt, L, P, 1.0 / np.sqrt(D))
    if gated:
        ref = Pr.output_gate(ref, bf16.to_f64(bits_of(gate)))
    assert_attn_close(out, ref)


def _layer_cases(n):
    out = []
    while len(out) < n:
        T = int(_rng.integers(1, 9))
        G = int(_rng.choice([1, 2, 4, 8, 16]))
        H_kv = int(_rng.integers(1, 3))
        D = int(_rng.choice([64, 128, 256]))
        R = int(_rng.choice([x for x in (16, 32, 64, 128, 256) if x <= D]))
        P = int(_rng.choice([16, 64]))
        lens = [int(x) for x in _rng.integers(T, 2500, int(_rng.integers(1, 3)))]
        out.append((len(out), T, G, H_kv, D, R, P, lens, bool(_rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _layer_cases(12), ids=lambda c: "layer%d" % c[0])
def test_random_fused_layer_shapes(case):
    i, T, G, H_kv, D, R, P, lens, gated = case
    seed = 8100 + i
    H_q = G * H_kv
    _, k_pool, v_pool, pt, L = paged_case(seed, lens, T, H_q, H_kv, D, P)
    S = len(lens)
    qg = synth.normal_bf16((S, T, H_q, 2, D), synth.seed_of(seed, 41))
    k = synth.normal_bf16((S, T, H_kv, D), synth.seed_of(seed, 42))
    v = synth.normal_bf16((S, T, H_kv, D), synth.seed_of(seed, 43))
    w_q = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 44))
    w_k = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 45))
    print("case %d: T=%d G=%d H_kv=%d D=%d R=%d P=%d lens=%s gated=%d" % (i, T, G, H_kv, D, R, P, lens, gated),
          flush=True)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, gate = had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt),
                                      to_dev(L), kd, vd, R, d_err=err, gated=gated)
    torch.cuda.synchronize()
    assert err.item() == 0
    kb_in, vb_in = bits_of(k_pool), bits_of(v_pool)
    for s in range(S):
        pos = np.arange(L[s] - T, L[s])
        q_ref, _, k_ref, v_ref = Pr.qk_norm_rope_gate(
            bf16.to_f64(bits_of(qg)[s]), bf16.to_f64(bits_of(k)[s]), bf16.to_f64(bits_of(v)[s]),
            w_q.numpy().astype(np.float64), w_k.numpy().astype(np.float64), pos, R)
        K = bf16.to_f64(PG.gather(kb_in, pt[s], L[s] - T, P))
        V = bf16.to_f64(PG.gather(vb_in, pt[s], L[s] - T, P))
        K = np.concatenate([K, bf16.to_f64(bf16.from_f64(k_ref))])
        V = np.concatenate([V, v_ref])
        ref = A.attention(bf16.to_f64(bf16.from_f64(q_ref)), K, V, 1.0 / np.sqrt(D))
        if gated:
            ref = Pr.output_gate(ref, bf16.to_f64(bits_of(qg)[s, :, :, 1]))
        assert_attn_close(out[s], ref)


def _prefill_cases(n, max_tokens=260, segmented=False):
    out = []
    for i in range(n):
        lens = [int(x) for x in _rng.integers(0, max_tokens, int(_rng.integers(1, 4)))]
        segs = int(_rng.integers(3, 9)) if segmented else 0
        out.append((i, lens, int(_rng.integers(1, 5)), int(_rng.choice([64, 128])), int(_rng.choice([64, 128])),
                    bool(_rng.integers(0, 2)), segs))
    return out


@pytest.mark.parametrize("case", _prefill_cases(10) + [(10 + c[0],) + c[1:] for c in _prefill_cases(5, 1600, True)],
                         ids=lambda c: "prefill%d" % c[0])
def test_random_gdn_prefill_shapes(case):
    i, lens, H, dk, dv, raw, segs = case
    seed = 8200 + i
    n = len(lens)
    N = max(1, sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = synth.l2_normalised_bf16((N, H, dk), synth.seed_of(seed, 1))
    k = synth.l2_normalised_bf16((N, H, dk), synth.seed_of(seed, 2))
    v = synth.normal_bf16((N, H, dv), synth.seed_of(seed, 3))
    if raw:
        a_in = -synth.uniform_f32((N, H), 0.0, 0.1, synth.seed_of(seed, 4))
        b_in = synth.uniform_f32((N, H), -3.0, 3.0, synth.seed_of(seed, 5))
        al, be = gdn.gates_from_raw(a_in.numpy(), b_in.numpy())
    else:
        a_in = synth.uniform_f32((N, H), 0.9, 1.0, synth.seed_of(seed, 4))
        b_in = synth.uniform_f32((N, H), 0.0, 1.0, synth.seed_of(seed, 5))
        al, be = a_in.numpy().astype(np.float64), b_in.numpy().astype(np.float64)
    n_slots = 2 * n + 1
    pool = synth.normal_f32((n_slots, H, dv, dk), synth.seed_of(seed, 6)) * 0.1
    in_idx = np.array([(2 * s + 1) if s % 2 else -1 for s in range(n)], np.int32)
    out_idx = np.array([2 * s for s in range(n)], np.int32)
    print("case %d: lens=%s H=%d dk=%d dv=%d raw=%d segments=%d" % (i, lens, H, dk, dv, raw, segs), flush=True)
    pd = to_dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = had.gdn_prefill(pd, to_dev(in_idx), to_dev(out_idx), to_dev(cu), to_dev(q), to_dev(k), to_dev(v),
                        to_dev(a_in), to_dev(b_in), max_len=max(max(lens), 1), d_err=err, raw_gates=raw,
                        n_segments=segs)
    torch.cuda.synchronize()
    assert err.item() == 0
    new_ref, o_ref = gdn.prefill(pool.numpy(), in_idx, out_idx, cu, bf16.to_f64(bits_of(q)), bf16.to_f64(bits_of(k)),
                                 bf16.to_f64(bits_of(v)), al, be)
    got = pd.cpu().numpy().astype(np.float64)
    for s in range(n):
        for h in range(H):
            ref = new_ref[out_idx[s], h].astype(np.float64)
            assert np.linalg.norm(got[out_idx[s], h] - ref) <= 1e-4 * max(np.linalg.norm(ref), 1e-30)
    oc = o.cpu().numpy().astype(np.float64)
    for t in range(int(cu[-1])):
        for h in range(H):
            assert np.linalg.norm(oc[t, h] - o_ref[t, h]) <= 1e-4 * max(np.linalg.norm(o_ref[t, h]), 1e-30)
