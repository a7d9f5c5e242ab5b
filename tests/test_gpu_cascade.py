"""GPU parity: shared-prefix (cascade) decode attention against the fp64
oracle and against the per-sequence split-K path."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import attention as A
from oracle import bf16
from oracle import paging as PG
from oracle import prologue as Pr
from gpu_util import DEV, assert_attn_close, bits_of, nan_bf16, to_dev

pytestmark = pytest.mark.gpu


def _batch(seed, n, prefix_len, suffixes, q_len, H_q, H_kv, D, P):
    """n sequences forked from one prefix (the oracle's page-table model), each
    with its own suffix + q_len new tokens; copy-on-write applied to the host
    pools; rows past every length hold NaN."""
    lens = [prefix_len + sfx + q_len for sfx in suffixes]
    max_pages = max(-(-L // P) for L in lens) + 1
    N = -(-prefix_len // P) + sum(-(-(sfx + q_len) // P) + 1 for sfx in suffixes) + 4
    order = synth.permutation(N, synth.seed_of(seed, 0))
    m = PG.PageTableModel(N, P, n + 1, max_pages, free_order=order)
    root = m.seq_create()
    m.reserve(root, prefix_len)
    kd = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 1))
    vd = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 2))
    seqs = []
    for i in range(n):
        sq = m.seq_fork(root, prefix_len)
        trip = m.reserve(sq, suffixes[i] + q_len)
        if trip is not None:
            kd[trip[1]] = kd[trip[0]]
            vd[trip[1]] = vd[trip[0]]
        seqs.append(sq)
    table, L = m.export(seqs, max_pages)
    # stale rows: NaN everywhere past each length in pages no sequence reads there
    kb, vb = kd.clone(), vd.clone()
    used = np.zeros((N, P), bool)
    for i in range(n):
        for t in range(int(L[i])):
            used[table[i, t // P], t % P] = True
    stale = torch.from_numpy(~used)
    kb[stale.nonzero(as_tuple=True)[0], :, stale.nonzero(as_tuple=True)[1]] = float("nan")
    vb[stale.nonzero(as_tuple=True)[0], :, stale.nonzero(as_tuple=True)[1]] = float("nan")
    q = synth.normal_bf16((n, q_len, H_q, D), synth.seed_of(seed, 3))
    prefix_pages = prefix_len // P
    assert np.all(table[:, :prefix_pages] == table[0, :prefix_pages])
    return q, kb, vb, table, L, table[0, :prefix_pages].copy()


def _oracle(q, kb, vb, table, L, P, D):
    kbits, vbits, qb = bits_of(kb), bits_of(vb), bf16.to_f64(bits_of(q))
    out = []
    for s in range(len(L)):
        K = bf16.to_f64(PG.gather(kbits, table[s], int(L[s]), P))
        V = bf16.to_f64(PG.gather(vbits, table[s], int(L[s]), P))
        out.append(A.attention(qb[s], K, V, 1.0 / np.sqrt(D)))
    return np.stack(out)


@pytest.mark.parametrize("n,prefix_len,q_len,H_q,H_kv,D,P", [
    (4, 1000, 1, 8, 1, 128, 16),     # 8 rows per sequence (VALU suffix), partial shared page copied
    (3, 2048, 4, 16, 1, 256, 64),    # speculative shape: 64 rows per sequence (MFMA suffix)
    (5, 700, 1, 4, 2, 64, 32),       # two KV heads
    (16, 5000, 1, 8, 1, 256, 64),    # prefix-shared batch shape (smaller prefix)
])
def test_cascade_matches_oracle(n, prefix_len, q_len, H_q, H_kv, D, P):
    seed = 3000 + n * 7 + prefix_len % 101
    suffixes = [int(x) for x in synth.integers(0, 3 * P + 5, n, synth.seed_of(seed, 9))]
    suffixes[0] = 0                                      # one sequence with no private token before the draft
    q, kb, vb, table, L, prefix = _batch(seed, n, prefix_len, suffixes, q_len, H_q, H_kv, D, P)
    print("case n=%d prefix=%d q_len=%d H_q=%d H_kv=%d D=%d P=%d suffixes=%s" % (
        n, prefix_len, q_len, H_q, H_kv, D, P, suffixes), flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kd, vd, pt, Ld = to_dev(kb), to_dev(vb), to_dev(table), to_dev(L)
    out = had.decode_attn_cascade(to_dev(q), kd, vd, pt, Ld, to_dev(prefix), d_err=err)
    ref_path = had.decode_attn(to_dev(q), kd, vd, pt, Ld)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = _oracle(q, kb, vb, table, L, P, D)
    assert_attn_close(out, ref)
    a, b = bf16.to_f64(bits_of(out)), bf16.to_f64(bits_of(ref_path))
    assert np.abs(a - b).max() <= 4e-3


def test_cascade_gated_output():
    n, prefix_len, q_len, H_q, H_kv, D, P = 6, 3000, 4, 16, 1, 256, 64
    seed = 3200
    suffixes = [int(x) for x in synth.integers(0, 3 * P + 5, n, synth.seed_of(seed, 9))]
    q, kb, vb, table, L, prefix = _batch(seed, n, prefix_len, suffixes, q_len, H_q, H_kv, D, P)
    gate = synth.normal_bf16(tuple(q.shape), synth.seed_of(seed, 8))
    print("case gated cascade n=%d prefix=%d suffixes=%s" % (n, prefix_len, suffixes), flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix),
                                  d_err=err, gate=to_dev(gate))
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = Pr.output_gate(_oracle(q, kb, vb, table, L, P, D), bf16.to_f64(bits_of(gate)))
    assert_attn_close(out, ref)


def test_cascade_sequence_inside_prefix_is_reported():
    n, prefix_len, P = 2, 512, 16
    q, kb, vb, table, L, prefix = _batch(3100, n, prefix_len, [5, 0], 1, 8, 1, 128, P)
    L = L.copy()
    L[1] = prefix_len - 3                                # this sequence does not see the whole prefix
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("case cascade with a too-short sequence", flush=True)
    had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix), d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_SEQLEN


def test_cascade_rejects_bad_prefix():
    q = torch.zeros((2, 1, 8, 128), dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros((8, 1, 16, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(had.HadError):
        had.decode_attn_cascade(q, pool, pool, torch.zeros((2, 4), dtype=torch.int32, device=DEV),
                                torch.tensor([40, 40], dtype=torch.int32, device=DEV),
                                torch.zeros(0, dtype=torch.int32, device=DEV))


def test_split_passes_and_one_call_cascade_match_the_oracle():
    # prefix pass, suffix pass and merge called one by one (the two-pass
    # layout) and had_decode_attn_cascade (here both passes in one launch,
    # units split on the device) each match the oracle, and the plan reports
    # the workspace's split counts
    P, D, H_q = 64, 256, 8
    q, kb, vb, table, L, prefix = _batch(4100, 5, 3200, [0, 700, 65, 1500, 9], 1, H_q, 1, D, P)
    print("case cascade split passes", flush=True)
    qd, kd, vd, ptd, ld, pxd = to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix)
    desc = had.attn_desc(q.shape, kb.shape, table.shape[1], deterministic=True)
    ns_p, ns_s = had.decode_attn_cascade_plan(desc, len(prefix))
    nbytes = had.decode_attn_cascade_workspace_bytes(desc, len(prefix))
    assert nbytes == len(L) * (ns_p + ns_s) * H_q * (D + 2) * 4
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    had.decode_attn_cascade_partial(qd, kd, vd, ptd, ld, pxd, ws, 1, d_err=err, deterministic=True)
    had.decode_attn_cascade_partial(qd, kd, vd, ptd, ld, pxd, ws, 2, d_err=err, deterministic=True)
    out = had.decode_attn_cascade_combine(qd, kd, vd, ptd, ld, pxd, ws, d_err=err, deterministic=True)
    one = had.decode_attn_cascade(qd, kd, vd, ptd, ld, pxd, d_err=err, deterministic=True)
    again = had.decode_attn_cascade(qd, kd, vd, ptd, ld, pxd, d_err=err, deterministic=True)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = _oracle(q, kb, vb, table, L, P, D)
    assert_attn_close(out, ref)
    assert_attn_close(one, ref)
    assert np.array_equal(bits_of(one), bits_of(again))      # deterministic mode: same bits every call
    with pytest.raises(had.HadError):
        had.decode_attn_cascade_partial(qd, kd, vd, ptd, ld, pxd, ws, 4)


@pytest.mark.parametrize("n,prefix_len,suffixes", [
    (16, 4096, [0] * 16),                       # only the decode tokens: few suffix tiles, most units to the prefix
    (9, 640, [9000] + [3] * 8),                 # one suffix much longer than the prefix: most units to it
    (2, 64 * 600, [1, 2]),                      # a prefix of 600 pages: at least 2 prefix units (page cap)
    (16, 2048, [int(x) for x in range(0, 16 * 700, 700)]),  # 128 prefix rows (the MFMA side that stages K and V straight into LDS)
])
def test_one_launch_cascade_unit_split(n, prefix_len, suffixes):
    # both passes in one grid: the prefix's share of the units follows its
    # share of the tiles, computed on the device from the lengths
    P, D, H_q = 64, 256, 8
    seed = 4200 + n + prefix_len % 89
    q, kb, vb, table, L, prefix = _batch(seed, n, prefix_len, suffixes, 1, H_q, 1, D, P)
    print("case one-launch cascade n=%d prefix=%d suffixes=%s" % (n, prefix_len, suffixes), flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix),
                                  d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert_attn_close(out, _oracle(q, kb, vb, table, L, P, D))


@pytest.mark.parametrize("n,prefix_len,H_q,H_kv,D,P,gated", [
    (6, 3000, 8, 1, 256, 64, True),     # gated output applied in the merge of the one-launch layout
    (4, 2048, 16, 2, 128, 64, False),   # two KV heads, 8 rows each, head_dim 128
    (3, 1280, 4, 1, 64, 32, True),      # 4 rows per sequence, 32-token pages
])
def test_one_launch_cascade_shapes(n, prefix_len, H_q, H_kv, D, P, gated):
    seed = 4300 + n * 11 + D
    suffixes = [int(x) for x in synth.integers(0, 6 * P, n, synth.seed_of(seed, 9))]
    q, kb, vb, table, L, prefix = _batch(seed, n, prefix_len, suffixes, 1, H_q, H_kv, D, P)
    gate = synth.normal_bf16(tuple(q.shape), synth.seed_of(seed, 8)) if gated else None
    print("case one-launch cascade n=%d prefix=%d H_q=%d H_kv=%d D=%d P=%d gated=%s suffixes=%s" % (
        n, prefix_len, H_q, H_kv, D, P, gated, suffixes), flush=True)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix),
                                  d_err=err, gate=to_dev(gate) if gated else None)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = _oracle(q, kb, vb, table, L, P, D)
    if gated:
        ref = Pr.output_gate(ref, bf16.to_f64(bits_of(gate)))
    assert_attn_close(out, ref)


def test_one_launch_cascade_reports_a_sequence_inside_the_prefix():
    n, prefix_len, P = 3, 1024, 64
    q, kb, vb, table, L, prefix = _batch(3150, n, prefix_len, [5, 0, 70], 1, 8, 1, 256, P)
    L = L.copy()
    L[1] = prefix_len - 3                                # this sequence does not see the whole prefix
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("case one-launch cascade with a too-short sequence", flush=True)
    out = had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix),
                                  d_err=err)
    torch.cuda.synchronize()
    assert err.item() & had.DERR_SEQLEN
    ref = _oracle(q[[0, 2]], kb, vb, table[[0, 2]], L[[0, 2]], P, 256)   # the others are unaffected
    assert_attn_close(out[[0, 2]], ref)


@pytest.mark.parametrize("n,spread,prefix_len,D,P", [
    (12, 6000, 3000, 256, 64),     # one long suffix among short ones: most units go to it
    (64, 900, 1000, 128, 16),      # as many sequences as the shares allow (one wave)
    (7, 0, 2048, 256, 64),         # only the decode tokens after the prefix
])
def test_cascade_suffix_units_by_length(n, spread, prefix_len, D, P):
    # the suffix pass shares its units out by suffix length (read from
    # seq_lens on the device) and the merge takes each sequence's own share
    seed = 3300 + n + spread % 97
    suffixes = [int(x) for x in synth.integers(0, max(spread // 8, 0), n, synth.seed_of(seed, 9))]
    if spread:
        suffixes[n // 2] = spread
    q, kb, vb, table, L, prefix = _batch(seed, n, prefix_len, suffixes, 1, 8, 1, D, P)
    print("case cascade units by length n=%d prefix=%d suffixes=%s" % (n, prefix_len, suffixes), flush=True)
    desc = had.attn_desc(q.shape, kb.shape, table.shape[1])
    assert had.decode_attn_cascade_plan(desc, len(prefix))[1] == max(n, 256)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = had.decode_attn_cascade(to_dev(q), to_dev(kb), to_dev(vb), to_dev(table), to_dev(L), to_dev(prefix),
                                  d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert_attn_close(out, _oracle(q, kb, vb, table, L, P, D))
