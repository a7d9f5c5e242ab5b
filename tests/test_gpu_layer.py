"""GPU parity: the fused attention layer (prologue inside the attention
kernel) against the fp64 oracle, and against the two-call path."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import attention as A
from oracle import bf16
from oracle import paging as PG
from oracle import prologue as Pr
from gpu_util import DEV, assert_attn_close, bits_of, paged_case, to_dev

pytestmark = pytest.mark.gpu


def _within_one_ulp(got_bits, ref):
    # one bf16 ulp of the exact value, plus the fp32 rounding of the row's
    # magnitude: the rotation y_i cos - y_j sin runs in fp32 on O(1) inputs,
    # so a result that cancels to ~1e-5 carries an absolute error of a few
    # fp32 ulps of its inputs, more than one bf16 ulp of itself
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    return np.all(np.abs(bf16.to_f64(got_bits) - ref) <= bf16.ulp(ref) + 2.0 ** -21 * scale)


def _inputs(seed, S, T, H_q, H_kv, D):
    qg = synth.normal_bf16((S, T, H_q, 2, D), synth.seed_of(seed, 41))
    k = synth.normal_bf16((S, T, H_kv, D), synth.seed_of(seed, 42))
    v = synth.normal_bf16((S, T, H_kv, D), synth.seed_of(seed, 43))
    w_q = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 44))
    w_k = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 45))
    return qg, k, v, w_q, w_k


def _run(seed, lens, T, H_q, H_kv, D, R, P, num_splits=0, deterministic=False, gated=False, max_seq_len=0):
    _, k_pool, v_pool, pt, L = paged_case(seed, lens, T, H_q, H_kv, D, P)
    qg, k, v, w_q, w_k = _inputs(seed, len(lens), T, H_q, H_kv, D)
    print("case seed=%d lens=%s T=%d H_q=%d H_kv=%d D=%d R=%d P=%d splits=%d gated=%d" % (
        seed, list(lens), T, H_q, H_kv, D, R, P, num_splits, gated), flush=True)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q_out = torch.empty((len(lens), T, H_q, D), dtype=torch.bfloat16, device=DEV)
    out, gate = had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt),
                                      to_dev(L), kd, vd, R, num_splits=num_splits, q_out=q_out, d_err=err,
                                      deterministic=deterministic, gated=gated, max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    assert err.item() == 0
    return dict(k_pool=k_pool, v_pool=v_pool, pt=pt, L=L, qg=qg, k=k, v=v, w_q=w_q, w_k=w_k, kd=kd, vd=vd,
                out=out, gate=gate, q_out=q_out, T=T, R=R, P=P, D=D, gated=gated)


def _check_against_oracle(c):
    T, R, P, D = c["T"], c["R"], c["P"], c["D"]
    kb_in, vb_in = bits_of(c["k_pool"]), bits_of(c["v_pool"])
    kb, vb = bits_of(c["kd"]), bits_of(c["vd"])
    touched = np.zeros(kb.shape[:1] + kb.shape[2:3], bool)
    for s, L in enumerate(c["L"]):
        pos = np.arange(L - T, L)
        q_ref, _, k_ref, v_ref = Pr.qk_norm_rope_gate(
            bf16.to_f64(bits_of(c["qg"])[s]), bf16.to_f64(bits_of(c["k"])[s]), bf16.to_f64(bits_of(c["v"])[s]),
            c["w_q"].numpy().astype(np.float64), c["w_k"].numpy().astype(np.float64), pos, R)
        assert _within_one_ulp(bits_of(c["q_out"])[s], q_ref)
        assert np.array_equal(bits_of(c["gate"])[s], bits_of(c["qg"])[s, :, :, 1])
        for j, p in enumerate(pos):
            page = c["pt"][s, p // P]
            touched[page, p % P] = True
            assert _within_one_ulp(kb[page, :, p % P], k_ref[j])
            assert np.array_equal(vb[page, :, p % P], bits_of(c["v"])[s, j])
        # attention over the prior context (pool input) + the oracle's new rows
        K = bf16.to_f64(PG.gather(kb_in, c["pt"][s], L - T, P))
        V = bf16.to_f64(PG.gather(vb_in, c["pt"][s], L - T, P))
        K = np.concatenate([K, bf16.to_f64(bf16.from_f64(k_ref))])
        V = np.concatenate([V, v_ref])
        ref = A.attention(bf16.to_f64(bf16.from_f64(q_ref)), K, V, 1.0 / np.sqrt(D))
        if c["gated"]:
            ref = Pr.output_gate(ref, bf16.to_f64(bits_of(c["qg"])[s, :, :, 1]))
        assert_attn_close(c["out"][s], ref)
    # nothing else in the pools changed
    for h in range(kb.shape[1]):
        assert np.array_equal(kb[:, h][~touched], kb_in[:, h][~touched], equal_nan=True)
        assert np.array_equal(vb[:, h][~touched], vb_in[:, h][~touched], equal_nan=True)


@pytest.mark.parametrize("lens,T,H_q,H_kv,D,R,P", [
    ([50001], 1, 8, 1, 256, 64, 64),          # the long-context layer shape (VALU, 8 rows)
    ([130, 1000], 2, 4, 1, 128, 32, 16),      # 8 rows, two sequences
    ([300], 3, 2, 1, 64, 16, 16),             # 6 rows
    ([4], 4, 2, 1, 128, 128, 16),             # the whole context is the new tokens
    ([7000], 4, 16, 1, 256, 64, 64),          # speculative verify shape (MFMA, 64 rows)
    ([97], 1, 16, 1, 128, 128, 16),           # 16 rows, one token
    ([2050, 513], 4, 8, 2, 64, 16, 64),       # 32 rows per KV head, two KV heads
    ([600], 4, 20, 1, 128, 32, 32),           # 80 rows: two MFMA row blocks
])
def test_fused_layer_matches_oracle(lens, T, H_q, H_kv, D, R, P):
    c = _run(2000 + sum(lens) % 997 + T, lens, T, H_q, H_kv, D, R, P)
    _check_against_oracle(c)


@pytest.mark.parametrize("H_q", [8, 16])
def test_new_tokens_straddle_splits(H_q):
    # one page per split and the 4 new tokens across a page boundary: two
    # splits hold new positions, the one with the last position owns them
    c = _run(2100 + H_q, [16 * 40 + 2], 4, H_q, 1, 128, 32, 16, num_splits=41)
    _check_against_oracle(c)


# The MFMA partial that loads K and V straight into LDS (pages of a
# multiple of 32 tokens; 16..64 rows at head_dim >= 128 with wave pairs,
# 65..128 rows with a wave per 16 rows): with the prologue inside it when
# the rotary dims are 0, 64 or a multiple of 128, else after the prologue
# kernel (32 rotary dims below)
@pytest.mark.parametrize("lens,T,H_q,H_kv,D,R,P", [
    ([3000, 41], 2, 16, 1, 128, 128, 32),     # 32 rows, whole head rotated, a 41-token sequence
    ([5000], 8, 8, 1, 256, 64, 96),           # 8 new tokens (one per wave), 96-token pages
    ([1000, 700], 4, 4, 1, 256, 256, 64),     # 16 rows: one wave pair
    ([900], 3, 16, 2, 128, 32, 32),           # 48 rows per KV head, two KV heads, 32 rotary dims (prologue kernel)
    ([32 * 10 + 3], 4, 16, 1, 256, 64, 32),   # the new tokens across a page boundary
    ([600], 4, 20, 1, 128, 64, 32),           # 80 rows, a wave per 16 rows
    ([400, 90], 8, 16, 1, 64, 64, 32),        # 128 rows at head_dim 64
    ([2000], 4, 16, 1, 256, 0, 64),           # no rotation
    ([700, 300], 2, 32, 2, 256, 128, 64),     # 64 rows per KV head, two KV heads, 128 rotary dims
    ([4, 300], 4, 16, 1, 128, 64, 32),        # a context of the new tokens only, next to a longer one
    ([97], 1, 16, 1, 128, 128, 32),           # 16 rows, one new token
])
def test_mfma_layer_matches_oracle(lens, T, H_q, H_kv, D, R, P):
    c = _run(3100 + sum(lens) % 997 + T, lens, T, H_q, H_kv, D, R, P)
    _check_against_oracle(c)


@pytest.mark.parametrize("num_splits", [1, 41, 300])
def test_mfma_layer_split_counts(num_splits):
    # one split; one 32-token stage per split with the 4 new tokens across
    # two splits; 300 splits, most of them empty
    c = _run(3200 + num_splits, [32 * 40 + 2], 4, 16, 1, 128, 64, 32, num_splits=num_splits)
    _check_against_oracle(c)


def test_mfma_layer_matches_two_call_path():
    lens, T, H_q, H_kv, D, R, P = [3000, 70], 4, 16, 1, 256, 64, 64
    c = _run(3300, lens, T, H_q, H_kv, D, R, P, deterministic=True)
    kd2, vd2 = to_dev(c["k_pool"]), to_dev(c["v_pool"])
    q2, g2 = had.qk_norm_rope_gate(to_dev(c["qg"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(c["w_q"]),
                                   to_dev(c["w_k"]), to_dev(c["pt"]), to_dev(c["L"]), kd2, vd2, R)
    out2 = had.decode_attn(q2, kd2, vd2, to_dev(c["pt"]), to_dev(c["L"]), deterministic=True)
    torch.cuda.synchronize()
    # the layer runs the prologue inside the MFMA partial (q rows in the
    # MFMA operand layout): the gate and the written pools agree bit for bit
    # (the keys use the prologue kernel's own row arithmetic); q within one
    # bf16 ulp, since the norm's fp32 sum of squares runs in another order
    qa, qb = bf16.to_f64(bits_of(c["q_out"])), bf16.to_f64(bits_of(q2))
    assert np.all(np.abs(qa - qb) <= bf16.ulp(qb))
    assert np.mean(qa != qb) < 0.01
    assert np.array_equal(bits_of(c["gate"]), bits_of(g2))
    assert np.array_equal(bits_of(c["kd"]), bits_of(kd2), equal_nan=True)
    assert np.array_equal(bits_of(c["vd"]), bits_of(vd2), equal_nan=True)
    a, b = bf16.to_f64(bits_of(c["out"])), bf16.to_f64(bits_of(out2))
    assert np.abs(a - b).max() <= 4e-3


@pytest.mark.parametrize("R", [32, 64])
def test_mfma_layer_bad_new_token_page_is_reported(R):
    # (R = 32: the prologue kernel; R = 64: the prologue inside the partial)
    _, k_pool, v_pool, pt, L = paged_case(3400, [200], 4, 16, 1, 128, 32)
    pt = pt.copy()
    pt[0, 199 // 32] = 10 ** 6                     # the page of the new tokens: out of range
    qg, k, v, w_q, w_k = _inputs(3400, 1, 4, 16, 1, 128)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    print("case bad new-token page (MFMA, 64 rows, R=%d)" % R, flush=True)
    had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt), to_dev(L),
                          kd, vd, R, d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_PAGE
    assert np.array_equal(bits_of(kd), bits_of(k_pool), equal_nan=True)   # nothing written
    assert np.array_equal(bits_of(vd), bits_of(v_pool), equal_nan=True)


@pytest.mark.parametrize("L,num_splits", [(666, 7), (643, 13), (700, 5)])
def test_valu_fused_tile_boundaries(L, num_splits):
    # 8 rows (2 q heads x 4 new tokens) on the fused VALU path, whose splits
    # are balanced to within one 8-token tile: boundaries fall inside pages
    # (96 tiles of 64-token pages over 7, 13 or 5 splits; over 7 splits the
    # first 5 take 14 tiles, the last 2 take 13), and with L = 666 and 7
    # splits the new tokens lie on both sides of one (tiles 82 | 83); the
    # split holding the last position's tile owns them
    c = _run(2150 + num_splits, [L], 4, 2, 1, 128, 32, 64, num_splits=num_splits)
    _check_against_oracle(c)


@pytest.mark.parametrize("lens,T,H_q,H_kv,D,R,P", [
    ([50001], 1, 8, 1, 256, 64, 64),          # VALU path
    ([7000, 300], 4, 16, 1, 256, 64, 64),     # MFMA path
    ([900], 2, 8, 2, 128, 32, 16),            # two KV heads
])
def test_gated_output_matches_oracle(lens, T, H_q, H_kv, D, R, P):
    c = _run(2500 + sum(lens) % 991 + T, lens, T, H_q, H_kv, D, R, P, gated=True)
    _check_against_oracle(c)


def test_gated_output_is_the_ungated_output_times_sigmoid():
    lens, T, H_q, H_kv, D, R, P = [3000], 1, 8, 1, 256, 64, 64
    a = _run(2600, lens, T, H_q, H_kv, D, R, P, deterministic=True)
    b = _run(2600, lens, T, H_q, H_kv, D, R, P, deterministic=True, gated=True)
    plain = bf16.to_f64(bits_of(a["out"]))
    gate = bf16.to_f64(bits_of(a["qg"])[:, :, :, 1])
    got = bf16.to_f64(bits_of(b["out"]))
    # same fp32 partials; the gate multiplies before the one rounding, so the
    # two differ by at most the ungated rounding (half an ulp) scaled, plus one
    assert np.all(np.abs(got - Pr.output_gate(plain, gate)) <= bf16.ulp(plain) + bf16.ulp(got))


def test_gated_flag_without_a_gate_is_rejected():
    q = torch.zeros((1, 1, 8, 128), dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros((4, 1, 16, 128), dtype=torch.bfloat16, device=DEV)
    desc = had._lib.attn_desc(q.shape, pool.shape, 4, gated=True)
    import ctypes
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    ptrs = had._lib.AttnPtrs(q.data_ptr(), pool.data_ptr(), pool.data_ptr(),
                             torch.zeros((1, 4), dtype=torch.int32, device=DEV).data_ptr(),
                             torch.tensor([20], dtype=torch.int32, device=DEV).data_ptr(), ws.data_ptr(), ws.numel(),
                             torch.empty_like(q).data_ptr(), None, None)
    assert had.lib().had_decode_attn(ctypes.byref(desc), ctypes.byref(ptrs), None) != 0
    # the split halves have no gate to apply, with or without the pointer
    ptrs.gate = q.data_ptr()
    assert had.lib().had_decode_attn_partial(ctypes.byref(desc), ctypes.byref(ptrs), None) != 0
    assert had.lib().had_decode_attn_combine(ctypes.byref(desc), 1, ws.data_ptr(), q.data_ptr(), None) != 0


def test_gated_two_call_path_matches_gated_layer():
    # prologue + decode_attn(gate=...) gives the fused layer's gated output
    lens, T, H_q, H_kv, D, R, P = [2500, 90], 2, 8, 1, 256, 64, 64
    c = _run(2700, lens, T, H_q, H_kv, D, R, P, deterministic=True, gated=True)
    _check_against_oracle(c)
    kd2, vd2 = to_dev(c["k_pool"]), to_dev(c["v_pool"])
    q2, g2 = had.qk_norm_rope_gate(to_dev(c["qg"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(c["w_q"]),
                                   to_dev(c["w_k"]), to_dev(c["pt"]), to_dev(c["L"]), kd2, vd2, R)
    out2 = had.decode_attn(q2, kd2, vd2, to_dev(c["pt"]), to_dev(c["L"]), deterministic=True, gate=g2)
    torch.cuda.synchronize()
    a, b = bf16.to_f64(bits_of(c["out"])), bf16.to_f64(bits_of(out2))
    assert np.abs(a - b).max() <= 4e-3


def test_fused_matches_two_call_path():
    lens, T, H_q, H_kv, D, R, P = [3000, 70], 2, 4, 1, 256, 64, 64
    c = _run(2200, lens, T, H_q, H_kv, D, R, P, deterministic=True)
    kd2, vd2 = to_dev(c["k_pool"]), to_dev(c["v_pool"])
    q2, g2 = had.qk_norm_rope_gate(to_dev(c["qg"]), to_dev(c["k"]), to_dev(c["v"]), to_dev(c["w_q"]),
                                   to_dev(c["w_k"]), to_dev(c["pt"]), to_dev(c["L"]), kd2, vd2, R)
    out2 = had.decode_attn(q2, kd2, vd2, to_dev(c["pt"]), to_dev(c["L"]), deterministic=True)
    torch.cuda.synchronize()
    # the layer runs the prologue inside the MFMA partial (q rows in the
    # MFMA operand layout): the gate and the written pools agree bit for bit
    # (the keys use the prologue kernel's own row arithmetic); q within one
    # bf16 ulp, since the norm's fp32 sum of squares runs in another order
    qa, qb = bf16.to_f64(bits_of(c["q_out"])), bf16.to_f64(bits_of(q2))
    assert np.all(np.abs(qa - qb) <= bf16.ulp(qb))
    assert np.mean(qa != qb) < 0.01
    assert np.array_equal(bits_of(c["gate"]), bits_of(g2))
    assert np.array_equal(bits_of(c["kd"]), bits_of(kd2), equal_nan=True)
    assert np.array_equal(bits_of(c["vd"]), bits_of(vd2), equal_nan=True)
    # the attention differs only in the order of its sums
    a, b = bf16.to_f64(bits_of(c["out"])), bf16.to_f64(bits_of(out2))
    assert np.abs(a - b).max() <= 4e-3


def test_bad_new_token_page_is_reported():
    _, k_pool, v_pool, pt, L = paged_case(2300, [200], 1, 8, 1, 128, 16)
    pt = pt.copy()
    pt[0, 199 // 16] = 10 ** 6                     # the page of the new token: out of range
    qg, k, v, w_q, w_k = _inputs(2300, 1, 1, 8, 1, 128)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("case bad new-token page", flush=True)
    had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt), to_dev(L),
                          to_dev(k_pool), to_dev(v_pool), 32, d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_PAGE


def test_disagreeing_descriptors_are_rejected():
    qg, k, v, w_q, w_k = _inputs(2400, 1, 9, 8, 1, 64)
    pool = torch.zeros((4, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(had.HadError) as e:
        had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k),
                              torch.zeros((1, 4), dtype=torch.int32, device=DEV),
                              torch.tensor([20], dtype=torch.int32, device=DEV), pool, pool.clone(), 16)
    assert e.value.kind == "unsupported_shape"          # T = 9 > 8


def test_split_touching_512_pages():
    # 4 rows, 64-token pages, 1532 planned pages over 3 splits: split 1's
    # tiles [4086, 8171) start and end inside pages 510 and 1021, so it reads
    # 512 page ids, the most a split holds; the context ends inside page 1531
    L = 1532 * 64 - 20
    c = _run(2800, [L], 1, 4, 1, 64, 16, 64, num_splits=3, max_seq_len=1532 * 64, gated=True)
    _check_against_oracle(c)


def test_length_beyond_the_split_plan_is_reported_and_writes_nothing():
    # max_seq_len bounds the plan (15 pages of 64 = 960 tokens); a length of
    # 1000 lies past it: the fused layer reports HAD_DERR_SEQLEN and neither
    # attends nor writes the new token's K/V
    _, k_pool, v_pool, pt, L = paged_case(2900, [1000], 1, 8, 1, 128, 64)
    qg, k, v, w_q, w_k = _inputs(2900, 1, 1, 8, 1, 128)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("case length past the plan (fused VALU)", flush=True)
    had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt), to_dev(L), kd, vd,
                          32, max_seq_len=900, d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_SEQLEN
    assert np.array_equal(bits_of(kd), bits_of(k_pool), equal_nan=True)
    assert np.array_equal(bits_of(vd), bits_of(v_pool), equal_nan=True)
    # the same on the MFMA path (64 rows; the prologue kernel at 32 rotary
    # dims, the prologue inside the partial at 64)
    for R in (32, 64):
        _, k_pool, v_pool, pt, L = paged_case(2902, [1000], 4, 16, 1, 128, 64)
        qg, k, v, w_q, w_k = _inputs(2902, 1, 4, 16, 1, 128)
        kd, vd = to_dev(k_pool), to_dev(v_pool)
        err.zero_()
        print("case length past the plan (MFMA layer, 64 rows, R=%d)" % R, flush=True)
        had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), to_dev(pt), to_dev(L), kd,
                              vd, R, max_seq_len=900, d_err=err)
        torch.cuda.synchronize()
        assert err.item() & had.DERR_SEQLEN
        assert np.array_equal(bits_of(kd), bits_of(k_pool), equal_nan=True)
        assert np.array_equal(bits_of(vd), bits_of(v_pool), equal_nan=True)
    # the plain call, VALU (8 rows) and MFMA (64 rows), reports it too
    for H_q, q_len in ((8, 1), (16, 4)):
        q, kp, vp, pt2, L2 = paged_case(2901 + H_q, [1000], q_len, H_q, 1, 128, 64)
        err.zero_()
        print("case length past the plan (decode_attn, %d rows)" % (H_q * q_len), flush=True)
        had.decode_attn(to_dev(q), to_dev(kp), to_dev(vp), to_dev(pt2), to_dev(L2), max_seq_len=900, d_err=err)
        torch.cuda.synchronize()
        assert err.item() & had.DERR_SEQLEN
