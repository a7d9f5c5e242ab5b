"""GPU parity: chunk-parallel GDN prefill vs the fp64 oracle (token-by-token
recurrence), and against the decode kernel run token by token."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import bf16, gdn
from gpu_util import DEV, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _rel_fro(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-30)


def _inputs(seed, N, H, dk, dv, alpha_lo=0.9):
    q = synth.l2_normalised_bf16((N, H, dk), synth.seed_of(seed, 1))
    k = synth.l2_normalised_bf16((N, H, dk), synth.seed_of(seed, 2))
    v = synth.normal_bf16((N, H, dv), synth.seed_of(seed, 3))
    al = synth.uniform_f32((N, H), alpha_lo, 1.0, synth.seed_of(seed, 4))
    be = synth.uniform_f32((N, H), 0.0, 1.0, synth.seed_of(seed, 5))
    return q, k, v, al, be


def _pool(seed, n_slots, H, dk, dv):
    # states of the size a warmed-up recurrence reaches (|S k| ~ |v|)
    return synth.normal_f32((n_slots, H, dv, dk), synth.seed_of(seed, 6)) * 0.1


def _run(seed, lens, H, dk, dv, in_idx, out_idx, n_slots, raw=False, q_scale=1.0, max_len=None, n_segments=0,
         alpha_lo=0.9):
    N = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, al, be = _inputs(seed, N, H, dk, dv, alpha_lo)
    if raw:  # raw gate values: the kernel forms exp(g) and sigmoid(b)
        al = -synth.uniform_f32((N, H), 0.0, 0.1, synth.seed_of(seed, 7))
        be = synth.uniform_f32((N, H), -3.0, 3.0, synth.seed_of(seed, 8))
    pool = _pool(seed, n_slots, H, dk, dv)
    print("case seed=%d lens=%s H=%d dk=%d dv=%d in=%s out=%s raw=%d segments=%d" % (
        seed, list(lens), H, dk, dv, in_idx, out_idx, raw, n_segments), flush=True)
    pd = to_dev(pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = had.gdn_prefill(pd, to_dev(np.asarray(in_idx, np.int32)), to_dev(np.asarray(out_idx, np.int32)), to_dev(cu),
                        to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be), max_len=max_len, q_scale=q_scale,
                        d_err=err, raw_gates=raw, n_segments=n_segments)
    torch.cuda.synchronize()
    alpha, beta = al.numpy().astype(np.float64), be.numpy().astype(np.float64)
    if raw:
        alpha, beta = gdn.gates_from_raw(alpha, beta)
    new_ref, o_ref = gdn.prefill(pool.numpy(), np.asarray(in_idx), np.asarray(out_idx), cu, bf16.to_f64(bits_of(q)),
                                 bf16.to_f64(bits_of(k)), bf16.to_f64(bits_of(v)), alpha, beta, q_scale)
    return dict(err=err.item(), got=pd.cpu().numpy(), o=o.cpu().numpy().astype(np.float64), new_ref=new_ref,
                o_ref=o_ref, pool=pool.numpy(), cu=cu, out_idx=out_idx, H=H)


def _check(c, tol=1e-4):
    assert c["err"] == 0
    written = set(int(x) for x in c["out_idx"])
    for sl in range(c["pool"].shape[0]):
        if sl in written:
            for h in range(c["H"]):
                assert _rel_fro(c["got"][sl, h].astype(np.float64), c["new_ref"][sl, h].astype(np.float64)) <= tol, \
                    (sl, h)
        else:
            assert np.array_equal(c["got"][sl], c["pool"][sl])   # untouched slots keep their bytes
    N = c["o"].shape[0]
    for t in range(N):
        for h in range(c["H"]):
            assert _rel_fro(c["o"][t, h], c["o_ref"][t, h]) <= tol, (t, h)


@pytest.mark.parametrize("lens,H,dk,dv", [
    ([1], 1, 64, 64),                  # one token
    ([64], 2, 128, 128),               # exactly one chunk
    ([65, 130], 2, 128, 128),          # ragged tails, two sequences
    ([200, 0, 37], 3, 64, 128),        # an empty sequence in the batch; d_k 64
    ([150], 2, 128, 64),               # d_v 64
    ([129, 3], 4, 64, 64),
])
def test_prefill_matches_oracle(lens, H, dk, dv):
    n = len(lens)
    in_idx = [-1] + [2 * i + 1 for i in range(1, n)]
    out_idx = [2 * i for i in range(n)]
    c = _run(4000 + sum(lens) + dk, lens, H, dk, dv, in_idx, out_idx, 2 * n + 1)
    _check(c)


def test_agentic_turn_800_tokens_8_heads():
    c = _run(4100, [800], 8, 128, 128, [3], [1], 4)
    _check(c)


def test_batch_of_turns_in_place_and_q_scale():
    # three sequences, one updating its slot in place; q_scale != 1
    c = _run(4200, [300, 511, 64], 8, 128, 128, [0, 5, -1], [0, 2, 3], 6, q_scale=0.088)
    _check(c)


def test_raw_gates():
    c = _run(4300, [333], 8, 128, 128, [2], [0], 3, raw=True)
    _check(c)


def test_loose_max_len_bound():
    # max_len well above the real lengths: chunks past a sequence do nothing
    c = _run(4400, [70, 10], 2, 128, 128, [1, 1], [0, 2], 3, max_len=1000)
    _check(c)


@pytest.mark.parametrize("lens,H,dk,dv,segs,max_len", [
    ([640], 2, 128, 128, 2, None),          # two segments of 5 chunks
    ([700, 77], 2, 128, 128, 3, None),      # ragged; the short sequence leaves segments empty
    ([1000], 1, 64, 128, 5, 1280),          # loose bound: the last segments are empty
    ([333, 0, 901], 2, 128, 64, 8, None),   # an empty sequence, d_v 64; one chunk per segment and less
    ([520], 3, 64, 64, 9, None),            # more segments than a sequence has chunks to spare
])
def test_segmented_scan_matches_oracle(lens, H, dk, dv, segs, max_len):
    n = len(lens)
    in_idx = [-1] + [2 * i + 1 for i in range(1, n)]
    out_idx = [2 * i for i in range(n)]
    c = _run(4700 + sum(lens) + segs, lens, H, dk, dv, in_idx, out_idx, 2 * n + 1, max_len=max_len,
             n_segments=segs)
    _check(c)


def test_segmented_scan_in_place_raw_gates():
    # segments with an in-place slot update (the link reads the input slot
    # before any segment writes the output slot) and raw gates
    c = _run(4800, [900, 450], 4, 128, 128, [2, 0], [2, 1], 3, raw=True, n_segments=4)
    _check(c)


def test_segmented_scan_weak_decay():
    # alpha in [0.999, 1]: the state keeps its history across segments, so
    # each segment's transition (near the identity) carries it and the link
    # is exercised, not just a state that has forgotten its start
    c = _run(4850, [1500], 2, 128, 128, [1], [0], 2, n_segments=6, alpha_lo=0.999)
    _check(c)


def test_segments_chosen_automatically_for_a_long_prompt():
    # one 6,144-token prompt with 2 heads: the plan segments the scan (3)
    desc = had.gdn_prefill_desc((2, 2, 128, 128), 1, 6144)
    one = had.gdn_prefill_desc((2, 2, 128, 128), 1, 6144, n_segments=1)
    assert had.gdn_prefill_workspace_bytes(desc) > had.gdn_prefill_workspace_bytes(one)
    c = _run(4900, [6144], 2, 128, 128, [0], [1], 2)
    _check(c)


def test_matches_decode_kernel_token_by_token():
    # the same 192 tokens through had_gdn_state_update one token at a time
    seed, T, H, dk, dv = 4500, 192, 8, 128, 128
    q, k, v, al, be = _inputs(seed, T, H, dk, dv)
    pool = _pool(seed, 3, H, dk, dv)
    p1, p2 = to_dev(pool), to_dev(pool)
    print("case prefill vs decode chain", flush=True)
    o1 = had.gdn_prefill(p1, to_dev(np.array([0], np.int32)), to_dev(np.array([1], np.int32)),
                         to_dev(np.array([0, T], np.int32)), to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be))
    qd, kd, vd, ad, bd = (to_dev(x) for x in (q, k, v, al, be))
    o2 = torch.empty((T, H, dv), dtype=torch.float32, device=DEV)
    slots = [0, 1, 2]
    for t in range(T):
        src, dst = (0, 1) if t == 0 else ((1, 2) if t % 2 else (2, 1))
        had.gdn_state_update(p2, to_dev(np.array([src], np.int32)), to_dev(np.array([[dst]], np.int32)),
                             qd[t:t + 1, None], kd[t:t + 1, None], vd[t:t + 1, None], ad[t:t + 1, None],
                             bd[t:t + 1, None], o=o2[t:t + 1, None])
    torch.cuda.synchronize()
    last = dst
    a = p1.cpu().numpy()[1].astype(np.float64)
    b = p2.cpu().numpy()[last].astype(np.float64)
    for h in range(H):
        assert _rel_fro(a[h], b[h]) <= 1e-4
    x, y = o1.cpu().numpy().astype(np.float64), o2.cpu().numpy().astype(np.float64)
    for t in range(T):
        for h in range(H):
            assert _rel_fro(x[t, h], y[t, h]) <= 1e-4
    del slots


def test_bad_slot_and_bad_length_are_reported():
    H, dk, dv = 1, 64, 64
    q, k, v, al, be = _inputs(4600, 10, H, dk, dv)
    pool = torch.zeros((2, H, dv, dk), dtype=torch.float32, device=DEV)
    for in_idx, out_idx, cu, max_len, bit in [([0], [5], [0, 10], 10, had.DERR_SLOT),
                                              ([-2], [1], [0, 10], 10, had.DERR_SLOT),
                                              ([0], [1], [0, 10], 8, had.DERR_SEQLEN)]:
        print("case bad in=%s out=%s max_len=%d" % (in_idx, out_idx, max_len), flush=True)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        had.gdn_prefill(pool, to_dev(np.array(in_idx, np.int32)), to_dev(np.array(out_idx, np.int32)),
                        to_dev(np.array(cu, np.int32)), to_dev(q), to_dev(k), to_dev(v), to_dev(al), to_dev(be),
                        max_len=max_len, d_err=err)
        torch.cuda.synchronize()
        assert err.item() & bit
    assert torch.count_nonzero(pool).item() == 0           # nothing written for a skipped sequence


def test_unsupported_head_dim_is_rejected():
    pool = torch.zeros((2, 1, 96, 96), dtype=torch.float32, device=DEV)
    x = torch.zeros((4, 1, 96), dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((4, 1), dtype=torch.float32, device=DEV)
    with pytest.raises(had.HadError):
        had.gdn_prefill(pool, to_dev(np.array([0], np.int32)), to_dev(np.array([1], np.int32)),
                        to_dev(np.array([0, 4], np.int32)), x, x, x, a, a)
