"""GPU parity: slot-addressed gated delta rule update vs the fp64 oracle."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import bf16, gdn
from gpu_util import DEV, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, S, T, H, dk, dv):
    q = synth.l2_normalised_bf16((S, T, H, dk), synth.seed_of(seed, 1))
    k = synth.l2_normalised_bf16((S, T, H, dk), synth.seed_of(seed, 2))
    v = synth.normal_bf16((S, T, H, dv), synth.seed_of(seed, 3))
    al = synth.uniform_f32((S, T, H), 0.9, 1.0, synth.seed_of(seed, 4))
    be = synth.uniform_f32((S, T, H), 0.0, 1.0, synth.seed_of(seed, 5))
    return q, k, v, al, be


def _warm_pool(seed, n_slots, H, dk, dv):
    """Initial states: the fp64 recurrence over 64 seeded warm-up tokens from 0."""
    pool = np.zeros((n_slots, H, dv, dk), np.float32)
    for sl in range(n_slots):
        q, k, v, al, be = _inputs(synth.seed_of(seed, 50, sl), 1, 64, H, dk, dv)
        for h in range(H):
            st, _ = gdn.sequential(np.zeros((dv, dk)), bf16.to_f64(bits_of(q)[0, :, h]), bf16.to_f64(bits_of(k)[0, :, h]),
                                   bf16.to_f64(bits_of(v)[0, :, h]), al.numpy()[0, :, h].astype(np.float64),
                                   be.numpy()[0, :, h].astype(np.float64))
            pool[sl, h] = st[-1].astype(np.float32)
    return pool


def _rel_fro(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-30)


def _run_and_check(seed, S, T, H, dk, dv, n_slots, in_idx, out_idx):
    pool = _warm_pool(seed, n_slots, H, dk, dv)
    q, k, v, al, be = _inputs(seed, S, T, H, dk, dv)
    print("case seed=%d S=%d T=%d H=%d dk=%d dv=%d in=%s out=%s" % (seed, S, T, H, dk, dv, in_idx, out_idx),
          flush=True)
    pd = to_dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = had.gdn_state_update(pd, to_dev(np.asarray(in_idx, np.int32)), to_dev(np.asarray(out_idx, np.int32)),
                             to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be), d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    new_ref, o_ref = gdn.state_update(pool, np.asarray(in_idx), np.asarray(out_idx), bf16.to_f64(bits_of(q)),
                                      bf16.to_f64(bits_of(k)), bf16.to_f64(bits_of(v)), al.numpy().astype(np.float64),
                                      be.numpy().astype(np.float64))
    got = pd.cpu().numpy()
    written = set(np.asarray(out_idx).ravel().tolist())
    for sl in range(n_slots):
        if sl in written:
            for h in range(H):
                assert _rel_fro(got[sl, h].astype(np.float64), new_ref[sl, h].astype(np.float64)) <= 1e-4
        else:
            assert np.array_equal(got[sl], pool[sl])   # untouched slots keep their bytes
    oc = o.cpu().numpy().astype(np.float64)
    for s in range(S):
        for t in range(T):
            for h in range(H):
                assert _rel_fro(oc[s, t, h], o_ref[s, t, h]) <= 1e-4


def test_tiny_config_single_head():
    _run_and_check(1, 1, 1, 1, 64, 64, 8, [3], [[6]])


def test_agentic_shape_8_heads_128():
    _run_and_check(2, 1, 1, 8, 128, 128, 4, [1], [[2]])


def test_speculative_checkpoints_t4():
    _run_and_check(3, 1, 4, 8, 128, 128, 8, [5], [[0, 7, 2, 3]])


def test_batch_with_shared_input_slot_and_zero_state():
    # two sequences read the same cached checkpoint (copy-on-write by index),
    # a third starts from the zero state
    _run_and_check(4, 3, 1, 2, 128, 64, 10, [4, 4, -1], [[1], [2], [9]])


# grids of 1024 waves or more run four waves per workgroup: a batch of 16
# sequences x 8 heads of 128 x 128 (permuted slots, as the prefix-shared
# batch), 4 drafts x 4 sequences, d_v 64 and d_k 64
@pytest.mark.parametrize("seed,S,T,H,dk,dv", [
    (11, 16, 1, 8, 128, 128),
    (12, 4, 4, 8, 128, 128),
    (13, 16, 1, 4, 128, 64),
    (14, 32, 1, 2, 64, 64),
])
def test_batch_grids_with_four_waves_per_workgroup(seed, S, T, H, dk, dv):
    assert S * H * (dv // 4) >= 1024
    n_slots = S * (T + 1) + 2
    perm = synth.permutation(n_slots, synth.seed_of(seed, 60))
    in_idx = perm[:S].tolist()
    out_idx = perm[S:S + S * T].reshape(S, T).tolist()
    _run_and_check(seed, S, T, H, dk, dv, n_slots, in_idx, out_idx)


def test_batch_grid_in_place_and_zero_states():
    # a grouped grid (16 x 8 x 32 waves) where every sequence writes the
    # slot it reads, two of them from the zero state (-1) into fresh slots
    S, H, dk, dv, n_slots = 16, 8, 128, 128, 20
    in_idx = list(range(S))
    out_idx = [[s] for s in range(S)]
    in_idx[3], out_idx[3] = -1, [17]
    in_idx[9], out_idx[9] = -1, [18]
    _run_and_check(15, S, 1, H, dk, dv, n_slots, in_idx, out_idx)


def test_in_place_single_token():
    _run_and_check(5, 1, 1, 2, 64, 128, 3, [1], [[1]])


def test_beta_zero_alpha_one_is_bit_exact_identity():
    H, dk, dv = 4, 128, 128
    pool = _warm_pool(6, 2, H, dk, dv)
    q, k, v, _, _ = _inputs(6, 1, 3, H, dk, dv)
    pd = to_dev(pool)
    ones = torch.ones((1, 3, H), dtype=torch.float32)
    zeros = torch.zeros((1, 3, H), dtype=torch.float32)
    had.gdn_state_update(pd, to_dev(np.array([0], np.int32)), to_dev(np.array([[1, 1, 1]], np.int32)), to_dev(q),
                         to_dev(k), to_dev(v), to_dev(ones), to_dev(zeros))
    torch.cuda.synchronize()
    assert np.array_equal(pd.cpu().numpy()[1], pool[0])


def test_bad_slot_sets_sentinel():
    H, dk, dv = 1, 64, 64
    pool = np.zeros((2, H, dv, dk), np.float32)
    q, k, v, al, be = _inputs(7, 1, 1, H, dk, dv)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pd = to_dev(pool)
    had.gdn_state_update(pd, to_dev(np.array([5], np.int32)), to_dev(np.array([[9]], np.int32)), to_dev(q), to_dev(k),
                         to_dev(v), to_dev(al), to_dev(be), d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_SLOT
    assert np.array_equal(pd.cpu().numpy(), pool)


def test_800_token_chain_drift():
    # free-running 800-step chain on the GPU (ping-pong between two slots)
    # against the fp64 recurrence: relative error <= 1e-3 at every step
    H, dk, dv, n = 8, 128, 128, 800
    pool = _warm_pool(8, 2, H, dk, dv)
    q, k, v, al, be = _inputs(8, 1, n, H, dk, dv)
    pd = to_dev(pool)
    qd, kd, vd, ad, bd = to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be)
    hist = torch.empty((n, H, dv, dk), dtype=torch.float32, device=DEV)
    for t in range(n):
        src, dst = t % 2, (t + 1) % 2
        had.gdn_state_update(pd, to_dev(np.array([src], np.int32)), to_dev(np.array([[dst]], np.int32)),
                             qd[:, t:t + 1].contiguous(), kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous(),
                             ad[:, t:t + 1].contiguous(), bd[:, t:t + 1].contiguous())
        hist[t].copy_(pd[dst])
    torch.cuda.synchronize()
    qf, kf, vf = bf16.to_f64(bits_of(q))[0], bf16.to_f64(bits_of(k))[0], bf16.to_f64(bits_of(v))[0]
    af, bfv = al.numpy()[0].astype(np.float64), be.numpy()[0].astype(np.float64)
    hh = hist.cpu().numpy().astype(np.float64)
    worst = 0.0
    for h in range(H):
        st, _ = gdn.sequential(pool[0, h].astype(np.float64), qf[:, h], kf[:, h], vf[:, h], af[:, h], bfv[:, h])
        for t in range(n):
            worst = max(worst, _rel_fro(hh[t, h], st[t]))
    print("worst relative state error over the chain: %.3g" % worst)
    assert worst <= 1e-3


def test_raw_gates_match_oracle_parameterisation():
    # the kernel forms alpha = exp(g), beta = sigmoid(b) from raw values
    seed, S, T, H, dk, dv, n_slots = 7, 2, 4, 8, 128, 128, 12
    pool = _warm_pool(seed, n_slots, H, dk, dv)
    q, k, v, _, _ = _inputs(seed, S, T, H, dk, dv)
    g = -synth.uniform_f32((S, T, H), 0.0, 0.1, synth.seed_of(seed, 6))
    b = synth.uniform_f32((S, T, H), -3.0, 3.0, synth.seed_of(seed, 7))
    in_idx, out_idx = [4, 9], [[0, 1, 2, 3], [5, 6, 7, 8]]
    print("case raw gates seed=%d S=%d T=%d" % (seed, S, T), flush=True)
    pd = to_dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = had.gdn_state_update(pd, to_dev(np.asarray(in_idx, np.int32)), to_dev(np.asarray(out_idx, np.int32)),
                             to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(b), d_err=err, raw_gates=True)
    torch.cuda.synchronize()
    assert err.item() == 0
    al, be = gdn.gates_from_raw(g.numpy(), b.numpy())
    new_ref, o_ref = gdn.state_update(pool, np.asarray(in_idx), np.asarray(out_idx), bf16.to_f64(bits_of(q)),
                                      bf16.to_f64(bits_of(k)), bf16.to_f64(bits_of(v)), al, be)
    got = pd.cpu().numpy()
    for sl in sorted(set(np.asarray(out_idx).ravel().tolist())):
        for h in range(H):
            assert _rel_fro(got[sl, h].astype(np.float64), new_ref[sl, h].astype(np.float64)) <= 1e-4
    oc = o.cpu().numpy().astype(np.float64)
    for s in range(S):
        for t in range(T):
            for h in range(H):
                assert _rel_fro(oc[s, t, h], o_ref[s, t, h]) <= 1e-4


def test_unknown_gdn_flag_is_rejected():
    pool = torch.zeros((2, 1, 64, 64), dtype=torch.float32, device=DEV)
    x = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((1, 1, 1), dtype=torch.float32, device=DEV)
    desc = had._lib.GdnDesc(1, 1, 1, 64, 64, 2, 1.0, 8)
    ptrs = had._lib.GdnPtrs(pool.data_ptr(), torch.zeros(1, dtype=torch.int32, device=DEV).data_ptr(),
                            torch.ones((1, 1), dtype=torch.int32, device=DEV).data_ptr(), x.data_ptr(), x.data_ptr(),
                            x.data_ptr(), a.data_ptr(), a.data_ptr(), torch.zeros((1, 1, 1, 64), device=DEV).data_ptr(),
                            None)
    import ctypes
    assert had.lib().had_gdn_state_update(ctypes.byref(desc), ctypes.byref(ptrs), None) != 0


def test_debug_mode_checks_slot_preconditions_on_the_host(monkeypatch):
    monkeypatch.setenv("HAD_DEBUG", "1")
    q, k, v, al, be = _inputs(8, 2, 1, 2, 64, 64)
    pool = torch.zeros((4, 2, 64, 64), dtype=torch.float32, device=DEV)
    print("case debug-mode slot checks", flush=True)
    had.gdn_state_update(pool, to_dev(np.array([0, 1], np.int32)), to_dev(np.array([[2], [3]], np.int32)),
                         to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be))
    torch.cuda.synchronize()
    with pytest.raises(had.HadError):   # slot 2 written by sequence 0 and read by sequence 1: never launched
        had.gdn_state_update(pool, to_dev(np.array([0, 2], np.int32)), to_dev(np.array([[2], [3]], np.int32)),
                             to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be))
