"""GPU parity at the full workload sizes the benchmark times.

Each test drives the library the way one decode step of the benchmark does
(same shapes, same default split plan, C++ page/slot bookkeeping) and checks
the results against the fp64 oracle on outputs it can afford: whole output
rows of one attention layer at 128K and 1M tokens, a speculative verify at
256K with rollback and the step after it, a 16-sequence prefix-shared batch
with copy-on-write, and a GDN + attention layer pair through the whole
agentic schedule (50,000-token first turn, 12 turns x 800 steps).

The prior context is seeded random data generated on the device and copied
to the host before any kernel runs; every later value the oracle uses (new
K/V rows, CoW copies, GDN states) it computes itself.
"""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import attention as A
from oracle import bf16, gdn
from oracle import paging as PG
from oracle import prologue as Pr
from gpu_util import DEV, assert_attn_close, bits_of, to_dev

pytestmark = pytest.mark.gpu

P, D, R, H_KV = 64, 256, 64, 1
GH, DK, DV = 8, 128, 128
BASE, EPS = 10000.0, 1e-6


def _say(*a):
    print(*a, flush=True)


def _round_bf16(x):
    return bf16.to_f64(bf16.from_f64(x))


def _rel_fro(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-30)


def _prologue_inputs(seed, S, T, H_q):
    qg = synth.normal_bf16((S, T, H_q, 2, D), synth.seed_of(seed, 1))
    k = synth.normal_bf16((S, T, H_KV, D), synth.seed_of(seed, 2))
    v = synth.normal_bf16((S, T, H_KV, D), synth.seed_of(seed, 3))
    w_q = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 4))
    w_k = synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 5))
    return qg, k, v, w_q, w_k


def _oracle_prologue(qg, k, v, w_q, w_k, s, positions):
    """Oracle q (bf16-rounded, as the cache and the kernels see it), k, v rows."""
    q_ref, _, k_ref, v_ref = Pr.qk_norm_rope_gate(
        bf16.to_f64(bits_of(qg)[s]), bf16.to_f64(bits_of(k)[s]), bf16.to_f64(bits_of(v)[s]),
        w_q.numpy().astype(np.float64), w_k.numpy().astype(np.float64), positions, R, BASE, EPS)
    return _round_bf16(q_ref), _round_bf16(k_ref), v_ref


def _gdn_inputs(seed, S, T):
    q = synth.l2_normalised_bf16((S, T, GH, DK), synth.seed_of(seed, 21))
    k = synth.l2_normalised_bf16((S, T, GH, DK), synth.seed_of(seed, 22))
    v = synth.normal_bf16((S, T, GH, DV), synth.seed_of(seed, 23))
    al = synth.uniform_f32((S, T, GH), 0.9, 1.0, synth.seed_of(seed, 24))
    be = synth.uniform_f32((S, T, GH), 0.0, 1.0, synth.seed_of(seed, 25))
    return q, k, v, al, be


def _gdn_f64(x):
    return bf16.to_f64(bits_of(x)) if x.dtype == torch.bfloat16 else x.numpy().astype(np.float64)


def _warm_state(seed):
    """Initial slot state: the recurrence over 64 seeded warm-up tokens from 0."""
    q, k, v, al, be = _gdn_inputs(synth.seed_of(seed, 60), 1, 64)
    S, _ = gdn.sequential_heads(np.zeros((GH, DV, DK)), _gdn_f64(q)[0], _gdn_f64(k)[0], _gdn_f64(v)[0],
                                _gdn_f64(al)[0], _gdn_f64(be)[0])
    return S.astype(np.float32)


def _pools(seed, N):
    kd = synth.normal_bf16((N, H_KV, P, D), synth.seed_of(seed, 30), device=DEV)
    vd = synth.normal_bf16((N, H_KV, P, D), synth.seed_of(seed, 31), device=DEV)
    torch.cuda.synchronize()
    return kd, vd, bits_of(kd), bits_of(vd)


def _context(kb, vb, pages, L):
    """fp64 [L, H_kv, D] K and V of positions 0..L-1 (oracle gather)."""
    return bf16.to_f64(PG.gather(kb, pages, L, P)), bf16.to_f64(PG.gather(vb, pages, L, P))


# ---------------------------------------------------------------- long context

@pytest.mark.parametrize("L0", [131072, 1048576])
def test_long_context_attention_layer(L0):
    """One attention layer of the long-context step at its full context."""
    seed, H_q, T = 300 + L0 % 97, 8, 1
    L = L0 + T
    n_pages = -(-L // P)
    N = n_pages + 4
    max_pages = -(-(L0 + 266) // P) + 1          # the benchmark's bound: 10 warm-up + 256 timed steps
    pages = synth.permutation(N, synth.seed_of(seed, 0))[:n_pages]
    pt = np.full((1, max_pages), -1, np.int32)
    pt[0, :n_pages] = pages
    _say("long-context layer L0=%d pages=%d" % (L0, n_pages))
    kd, vd, kb, vb = _pools(seed, N)
    qg, k, v, w_q, w_k = _prologue_inputs(seed, 1, T, H_q)
    pt_d, lens_d = to_dev(pt), to_dev(np.array([L], np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q_out, _ = had.qk_norm_rope_gate(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), pt_d, lens_d, kd, vd,
                                     R, BASE, EPS, d_err=err)
    out = had.decode_attn(q_out, kd, vd, pt_d, lens_d, max_seq_len=L0 + 266, d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    q_ref, k_new, v_new = _oracle_prologue(qg, k, v, w_q, w_k, 0, [L0])
    K, V = _context(kb, vb, pages, L0)
    K = np.concatenate([K, k_new], 0)
    V = np.concatenate([V, v_new], 0)
    ref = A.attention(q_ref, K, V, 1.0 / np.sqrt(D))
    assert_attn_close(out[0], ref)


# The benchmark's launch: bench.py's long-context step calls
# had_decode_attn_layer (prologue fused into the VALU partial kernel, gated
# output) with max_seq_len = L0 + warmup + steps + 2, which fixes the split
# plan (256 splits, tile ranges inside 9 / 17 / 65-page spans).  Its default
# run (10 + 256 steps) and a short run (5 + 20 steps) give different plans.
@pytest.mark.parametrize("L0,extra,at", [
    (131072, 268, 1), (131072, 268, 268), (131072, 27, 27), (262144, 268, 1), (1048576, 268, 1)])
def test_long_context_fused_gated_layer_bench_plan(L0, extra, at):
    seed, H_q, T = 350 + L0 % 89 + at, 8, 1
    L = L0 + at                                  # the decode token at position L - 1
    max_len = L0 + extra
    n_pages = -(-L // P)
    max_pages = -(-max_len // P) + 1             # as the benchmark's stack
    N = max_pages + 4
    pages = synth.permutation(N, synth.seed_of(seed, 0))[:n_pages]
    pt = np.full((1, max_pages), -1, np.int32)
    pt[0, :n_pages] = pages
    desc = had.attn_desc((1, 1, H_q, D), (N, H_KV, P, D), max_pages, max_seq_len=max_len, gated=True)
    ns, pps = had.decode_attn_plan(desc)
    _say("fused gated layer L0=%d L=%d plan: %d splits, %d pages per split" % (L0, L, ns, pps))
    assert ns == 256
    kd, vd, kb, vb = _pools(seed, N)
    qg, k, v, w_q, w_k = _prologue_inputs(seed, 1, T, H_q)
    pt_d, lens_d = to_dev(pt), to_dev(np.array([L], np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(had.decode_attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 1, H_q, D), dtype=torch.bfloat16, device=DEV)
    gate = torch.empty_like(out)
    q_out = torch.empty_like(out)
    had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), pt_d, lens_d, kd, vd, R,
                          max_seq_len=max_len, workspace=ws, out=out, gate_out=gate, q_out=q_out, d_err=err,
                          gated=True)
    torch.cuda.synchronize()
    assert err.item() == 0
    q_ref, k_new, v_new = _oracle_prologue(qg, k, v, w_q, w_k, 0, [L - 1])
    # q and the new K/V row (within 1 bf16 ulp of the fp64 value; v and the gate bit-exact)
    assert np.all(np.abs(bf16.to_f64(bits_of(q_out)[0]) - q_ref) <= bf16.ulp(q_ref))
    assert np.array_equal(bits_of(gate)[0], bits_of(qg)[0, :, :, 1])
    page, row = pages[(L - 1) // P], (L - 1) % P
    kb_after, vb_after = bits_of(kd), bits_of(vd)
    assert np.all(np.abs(bf16.to_f64(kb_after[page, :, row]) - k_new[0]) <= bf16.ulp(k_new[0]))
    assert np.array_equal(vb_after[page, :, row], bits_of(v)[0, 0])
    kb_after[page, :, row] = kb[page, :, row]
    vb_after[page, :, row] = vb[page, :, row]
    assert np.array_equal(kb_after, kb) and np.array_equal(vb_after, vb)      # nothing else written
    K, V = _context(kb, vb, pages, L - 1)
    ref = A.attention(q_ref, np.concatenate([K, k_new]), np.concatenate([V, v_new]), 1.0 / np.sqrt(D))
    ref = Pr.output_gate(ref, bf16.to_f64(bits_of(qg)[0, :, :, 1]))
    assert_attn_close(out[0], ref)


# ---------------------------------------------------------------- speculative

def test_speculative_verify_rollback_256k():
    """Verify 4 drafts at 256K (64 query rows, MFMA path) with GDN
    checkpoints, keep 2 (rollback by index), then decode one token: results
    equal an oracle run that never saw the rejected drafts."""
    seed, H_q, T, L0, acc = 400, 16, 4, 262144, 2
    max_pages = -(-(L0 + 2 * T) // P) + 1
    N = max_pages + 4
    n_slots = 2 * T + 2
    pt = had.PageTable(N, P, 1, max_pages, free_order=synth.permutation(N, synth.seed_of(seed, 0)))
    slots = had.SlotPool(n_slots, free_order=synth.permutation(n_slots, synth.seed_of(seed, 1)))
    sq = pt.seq_create()
    pt.reserve(sq, L0)
    cur = slots.acquire()
    _say("speculative 256K: verify T=4")
    kd, vd, kb, vb = _pools(seed, N)
    pool0 = np.zeros((n_slots, GH, DV, DK), np.float32)
    pool0[cur] = _warm_state(seed)
    pool_d = to_dev(pool0)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scale = 1.0 / np.sqrt(D)

    # ---- step 1: T drafts
    assert pt.reserve(sq, T) is None
    table, lens = pt.export([sq], max_pages)
    pages1 = table[0].copy()
    outs = [slots.acquire() for _ in range(T)]
    qg, k, v, w_q, w_k = _prologue_inputs(seed, 1, T, H_q)
    gq, gk, gv, gal, gbe = _gdn_inputs(seed, 1, T)
    pt_d, lens_d = to_dev(table), to_dev(lens)
    # the benchmark's call: had_decode_attn_layer with the prologue inside
    # the MFMA partial, gated output, 256 splits
    q_out = torch.empty((1, T, H_q, D), dtype=torch.bfloat16, device=DEV)
    out1, gate1 = had.decode_attn_layer(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), pt_d, lens_d, kd,
                                        vd, R, BASE, EPS, max_seq_len=L0 + 2 * T, q_out=q_out, d_err=err, gated=True)
    o1 = had.gdn_state_update(pool_d, to_dev(np.array([cur], np.int32)), to_dev(np.array([outs], np.int32)),
                              to_dev(gq), to_dev(gk), to_dev(gv), to_dev(gal), to_dev(gbe), d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert had.decode_attn_plan(had.attn_desc((1, T, H_q, D), tuple(kd.shape), max_pages, max_seq_len=L0 + 2 * T,
                                              gated=True))[0] == 256
    ckpt = pool_d.cpu().numpy()

    q_ref, k_new, v_new = _oracle_prologue(qg, k, v, w_q, w_k, 0, np.arange(L0, L0 + T))
    # q, the gate and the new K/V rows (q and k within 1 bf16 ulp of the fp64
    # value, the gate and v bit-exact)
    assert np.all(np.abs(bf16.to_f64(bits_of(q_out)[0]) - q_ref) <= bf16.ulp(q_ref))
    assert np.array_equal(bits_of(gate1)[0], bits_of(qg)[0, :, :, 1])
    kb1, vb1 = bits_of(kd), bits_of(vd)
    for t in range(T):
        page, row = pages1[(L0 + t) // P], (L0 + t) % P
        assert np.all(np.abs(bf16.to_f64(kb1[page, :, row]) - k_new[t]) <= bf16.ulp(k_new[t]))
        assert np.array_equal(vb1[page, :, row], bits_of(v)[0, t])
    K0, V0 = _context(kb, vb, pages1, L0)
    ref1 = A.attention(q_ref, np.concatenate([K0, k_new]), np.concatenate([V0, v_new]), scale)
    assert_attn_close(out1[0], Pr.output_gate(ref1, bf16.to_f64(bits_of(qg)[0, :, :, 1])))
    S = pool0[cur].astype(np.float64)
    for t in range(T):
        S, o_ref = gdn.sequential_heads(S, _gdn_f64(gq)[0, t:t + 1], _gdn_f64(gk)[0, t:t + 1], _gdn_f64(gv)[0, t:t + 1],
                                        _gdn_f64(gal)[0, t:t + 1], _gdn_f64(gbe)[0, t:t + 1])
        for h in range(GH):
            assert _rel_fro(ckpt[outs[t], h].astype(np.float64), S[h]) <= 1e-4
            assert _rel_fro(o1.cpu().numpy()[0, t, h].astype(np.float64), o_ref[0, h]) <= 1e-4
        if t == acc - 1:
            S_acc = S.copy()

    # ---- accept 2 drafts: rollback by index
    cur2 = had.spec_rollback(pt, slots, sq, T, acc, cur, outs)
    assert cur2 == outs[acc - 1]
    assert pt.seq_len(sq) == L0 + acc

    # ---- step 2: one token at position L0 + acc; the rejected draft at
    # L0 + acc + 1 stays in the page as stale data and must stay invisible
    _say("speculative 256K: decode after rollback")
    assert pt.reserve(sq, 1) is None
    table2, lens2 = pt.export([sq], max_pages)
    out2_slot = slots.acquire()
    qg2, k2, v2, _, _ = _prologue_inputs(seed + 1, 1, 1, H_q)
    gq2, gk2, gv2, gal2, gbe2 = _gdn_inputs(seed + 1, 1, 1)
    pt_d, lens_d = to_dev(table2), to_dev(lens2)
    q_out2, _ = had.qk_norm_rope_gate(to_dev(qg2), to_dev(k2), to_dev(v2), to_dev(w_q), to_dev(w_k), pt_d, lens_d, kd,
                                      vd, R, BASE, EPS, d_err=err)
    out2 = had.decode_attn(q_out2, kd, vd, pt_d, lens_d, max_seq_len=L0 + 2 * T, d_err=err)
    o2 = had.gdn_state_update(pool_d, to_dev(np.array([cur2], np.int32)), to_dev(np.array([[out2_slot]], np.int32)),
                              to_dev(gq2), to_dev(gk2), to_dev(gv2), to_dev(gal2), to_dev(gbe2), d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0

    # the never-drafted oracle run: prior context + the 2 kept drafts + the new token
    q_ref2, k_new2, v_new2 = _oracle_prologue(qg2, k2, v2, w_q, w_k, 0, [L0 + acc])
    K = np.concatenate([K0, k_new[:acc], k_new2])
    V = np.concatenate([V0, v_new[:acc], v_new2])
    ref2 = A.attention(q_ref2, K, V, scale)
    assert_attn_close(out2[0], ref2)
    S2, o2_ref = gdn.sequential_heads(S_acc, _gdn_f64(gq2)[0], _gdn_f64(gk2)[0], _gdn_f64(gv2)[0], _gdn_f64(gal2)[0],
                                      _gdn_f64(gbe2)[0])
    got = pool_d.cpu().numpy()[out2_slot]
    for h in range(GH):
        assert _rel_fro(got[h].astype(np.float64), S2[h]) <= 1e-4
        assert _rel_fro(o2.cpu().numpy()[0, 0, h].astype(np.float64), o2_ref[0, h]) <= 1e-4


# ---------------------------------------------------------------- prefix-shared

def test_prefix_shared_batch_copy_on_write():
    """16 sequences fork a 50,000-token prefix, take private suffixes of
    U{0..12288} tokens and decode one token each: shared pages are read
    through every sequence's page table (and, by the cascade path, once for
    all sequences), the shared partial page is copied on first write, and
    GDN states come from permuted slots (sequences with no suffix read the
    shared prefix checkpoint)."""
    seed, n, prefix, H_q, n_slots = 500, 16, 50000, 8, 64
    suffix = synth.integers(0, 12288, n, synth.seed_of(seed, 2))
    suffix[3] = 0                                            # at least one sequence without a suffix
    max_pages = -(-(prefix + int(suffix.max()) + 2) // P) + 1
    N = -(-prefix // P) + sum(-(-(int(x) + 2) // P) + 1 for x in suffix) + 8
    order = synth.permutation(N, synth.seed_of(seed, 0))
    pt = had.PageTable(N, P, n + 1, max_pages, free_order=order)
    model = PG.PageTableModel(N, P, n + 1, max_pages, free_order=order)
    _say("prefix-shared batch: 16 sequences, suffixes %s" % [int(x) for x in suffix])
    kd, vd, kb, vb = _pools(seed, N)
    kb_ref, vb_ref = kb.copy(), vb.copy()
    root, mroot = pt.seq_create(), model.seq_create()
    pt.reserve(root, prefix)
    model.reserve(mroot, prefix)
    seqs = [pt.seq_fork(root, prefix) for _ in range(n)]
    mseqs = [model.seq_fork(mroot, prefix) for _ in range(n)]

    def grow(s, m, count):
        trip, mtrip = pt.reserve(s, count), model.reserve(m, count)
        if mtrip is not None:                                # oracle: copy the whole page
            kb_ref[mtrip[1]] = kb_ref[mtrip[0]]
            vb_ref[mtrip[1]] = vb_ref[mtrip[0]]
        if trip is not None:
            had.kv_copy_pages(kd, vd, [trip[0]], [trip[1]])

    for i in range(n):
        if suffix[i] > 0:
            grow(seqs[i], mseqs[i], int(suffix[i]))
    for i in range(n):                                       # the decode token
        grow(seqs[i], mseqs[i], 1)
    table, lens = pt.export(seqs, max_pages)
    mtable, mlens = model.export(mseqs, max_pages)
    assert np.array_equal(table, mtable) and np.array_equal(lens, mlens)

    # GDN: permuted slots; sequences without a suffix share the prefix checkpoint
    slot_order = synth.permutation(n_slots, synth.seed_of(seed, 3))
    slots = had.SlotPool(n_slots, free_order=slot_order)
    shared = slots.acquire()
    in_idx = []
    for i in range(n):
        if suffix[i] == 0:
            slots.retain(shared)
            in_idx.append(shared)
        else:
            in_idx.append(slots.acquire())
    out_idx = [[slots.acquire()] for _ in range(n)]
    pool0 = np.zeros((n_slots, GH, DV, DK), np.float32)
    for sl in set(in_idx):
        pool0[sl] = _warm_state(synth.seed_of(seed, 70, sl))
    pool_d = to_dev(pool0)

    qg, k, v, w_q, w_k = _prologue_inputs(seed, n, 1, H_q)
    gq, gk, gv, gal, gbe = _gdn_inputs(seed, n, 1)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pt_d, lens_d = to_dev(table), to_dev(lens)
    q_out, _ = had.qk_norm_rope_gate(to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k), pt_d, lens_d, kd, vd,
                                     R, BASE, EPS, d_err=err)
    out = had.decode_attn(q_out, kd, vd, pt_d, lens_d, max_seq_len=int(lens.max()), d_err=err)
    # the same attention with the prefix's whole pages read once for all sequences
    out_c = had.decode_attn_cascade(q_out, kd, vd, pt_d, lens_d, to_dev(mtable[0, :prefix // P].copy()),
                                    max_seq_len=int(lens.max()), d_err=err)
    o = had.gdn_state_update(pool_d, to_dev(np.array(in_idx, np.int32)), to_dev(np.array(out_idx, np.int32)),
                             to_dev(gq), to_dev(gk), to_dev(gv), to_dev(gal), to_dev(gbe), d_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0

    # pages the prefix still shares are untouched; sampled sequences' outputs
    kb_after = bits_of(kd)
    shared_pages = [p for p in mtable[0][:prefix // P] if p >= 0]
    assert np.array_equal(kb_after[shared_pages], kb[shared_pages])
    scale = 1.0 / np.sqrt(D)
    sample = sorted({3, int(np.argmax(suffix)), 0, n - 1})
    for i in sample:
        L = int(lens[i])
        q_ref, k_new, v_new = _oracle_prologue(qg, k, v, w_q, w_k, i, [L - 1])
        K, V = _context(kb_ref, vb_ref, mtable[i], L - 1)
        ref = A.attention(q_ref, np.concatenate([K, k_new]), np.concatenate([V, v_new]), scale)
        assert_attn_close(out[i], ref)
        assert_attn_close(out_c[i], ref)
    new_pool, o_ref = gdn.state_update(pool0, np.array(in_idx), np.array(out_idx), _gdn_f64(gq), _gdn_f64(gk),
                                       _gdn_f64(gv), _gdn_f64(gal), _gdn_f64(gbe))
    got = pool_d.cpu().numpy()
    for i in range(n):
        sl = out_idx[i][0]
        for h in range(GH):
            assert _rel_fro(got[sl, h].astype(np.float64), new_pool[sl, h].astype(np.float64)) <= 1e-4
            assert _rel_fro(o.cpu().numpy()[i, 0, h].astype(np.float64), o_ref[i, 0, h]) <= 1e-4
    assert np.array_equal(got[shared], pool0[shared])       # the shared checkpoint is never written


# ---------------------------------------------------------------- agentic

def test_agentic_schedule_turn_checkpoints():
    """One attention + one GDN layer through the agentic schedule: a
    50,000-token first turn, then 12 turns x 800 decode steps.  At every turn
    boundary the current GDN slot is kept as a checkpoint; each kept
    checkpoint must still hold the state at its boundary at the end, and the
    attention output is checked at the first step, at the last step of the
    first turn and at the final step."""
    seed, H_q, first, turns, per = 600, 8, 50000, 12, 800
    steps = turns * per
    max_pages = -(-(first + steps + 1) // P) + 1
    N = max_pages + 4
    pt = had.PageTable(N, P, 1, max_pages, free_order=synth.permutation(N, synth.seed_of(seed, 0)))
    slots = had.SlotPool(turns + 4, free_order=synth.permutation(turns + 4, synth.seed_of(seed, 1)))
    sq = pt.seq_create()
    pt.reserve(sq, first)
    _say("agentic schedule: %d + %d x %d steps" % (first, turns, per))
    kd, vd, kb, vb = _pools(seed, N)
    cur = cur0 = slots.acquire()
    pool0 = np.zeros((turns + 4, GH, DV, DK), np.float32)
    pool0[cur] = _warm_state(seed)
    pool_d = to_dev(pool0)
    qg, k, v, w_q, w_k = _prologue_inputs(seed, steps, 1, H_q)     # one row per step
    gq, gk, gv, gal, gbe = _gdn_inputs(seed, steps, 1)
    qg_d, k_d, v_d, wq_d, wk_d = to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k)
    gdn_d = [to_dev(x) for x in (gq, gk, gv, gal, gbe)]
    table, _ = pt.export([sq], max_pages)
    pt_d = to_dev(table)
    lens_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    in_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    out_d = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = had.attn_desc((1, 1, H_q, D), kd.shape, max_pages, max_seq_len=first + steps + 1)
    ws = torch.empty(had.decode_attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    checkpoints, sampled = [], {}
    check_at = {0, per - 1, steps - 1}
    for t in range(steps):
        if t > 0 and t % per == 0:
            slots.retain(cur)
            checkpoints.append((t, cur))
        out_slot = slots.acquire()
        assert pt.reserve(sq, 1) is None
        L = first + t + 1
        if (L - 1) % P == 0:
            table, _ = pt.export([sq], max_pages)
            pt_d.copy_(torch.from_numpy(table))
        lens_d.fill_(L)
        in_d.fill_(cur)
        out_d.fill_(out_slot)
        q_out, _ = had.qk_norm_rope_gate(qg_d[t:t + 1], k_d[t:t + 1], v_d[t:t + 1], wq_d, wk_d, pt_d, lens_d, kd, vd,
                                         R, BASE, EPS, d_err=err)
        o = had.decode_attn(q_out, kd, vd, pt_d, lens_d, max_seq_len=first + steps + 1, workspace=ws, d_err=err)
        had.gdn_state_update(pool_d, in_d, out_d, *[x[t:t + 1] for x in gdn_d], d_err=err)
        if t in check_at:
            sampled[t] = o.clone()
        slots.release(cur)
        cur = out_slot
    torch.cuda.synchronize()
    assert err.item() == 0
    got_pool = pool_d.cpu().numpy()
    table, _ = pt.export([sq], max_pages)

    # oracle: every decode row's k (prologue), then attention at the sampled steps
    _, k_rows, v_rows = _oracle_prologue(
        qg.reshape(1, steps, H_q, 2, D), k.reshape(1, steps, H_KV, D), v.reshape(1, steps, H_KV, D), w_q, w_k, 0,
        np.arange(first, first + steps))
    K0, V0 = _context(kb, vb, table[0], first)
    scale = 1.0 / np.sqrt(D)
    for t, o in sampled.items():
        q_ref, _, _ = _oracle_prologue(qg, k, v, w_q, w_k, t, [first + t])
        K = np.concatenate([K0, k_rows[:t + 1]])
        V = np.concatenate([V0, v_rows[:t + 1]])
        assert_attn_close(o[0], A.attention(q_ref, K, V, scale))

    # oracle: the GDN chain in fp64, compared with every kept checkpoint and the final state
    S = pool0[cur0].astype(np.float64)
    f = [_gdn_f64(x)[:, 0] for x in (gq, gk, gv, gal, gbe)]
    done = 0
    for t_b, slot in checkpoints + [(steps, cur)]:
        S, _ = gdn.sequential_heads(S, *[x[done:t_b] for x in f])
        done = t_b
        for h in range(GH):
            assert _rel_fro(got_pool[slot, h].astype(np.float64), S[h]) <= 1e-3, (t_b, h)


@pytest.mark.timeout(400)   # the fp64 oracle walks 50,000 tokens one by one (~40 s)
def test_gdn_prefill_first_turn_50k():
    # the agentic workload's 50,000-token first turn through one GDN layer
    # (8 heads, d_k = d_v = 128) by the chunk-parallel prefill, against the
    # token-by-token fp64 recurrence: the final state of every head and the
    # outputs of a spread of tokens
    N = 50000
    q = synth.l2_normalised_bf16((N, GH, DK), synth.seed_of(910, 1))
    k = synth.l2_normalised_bf16((N, GH, DK), synth.seed_of(910, 2))
    v = synth.normal_bf16((N, GH, DV), synth.seed_of(910, 3))
    g = -synth.uniform_f32((N, GH), 0.0, 0.1, synth.seed_of(910, 4))   # raw gates, as the model feeds them
    b = synth.uniform_f32((N, GH), -3.0, 3.0, synth.seed_of(910, 5))
    pool = torch.zeros((2, GH, DV, DK), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _say("case gdn prefill 50k first turn")
    o = had.gdn_prefill(pool, to_dev(np.array([-1], np.int32)), to_dev(np.array([1], np.int32)),
                        to_dev(np.array([0, N], np.int32)), to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(b),
                        d_err=err, raw_gates=True)
    torch.cuda.synchronize()
    assert err.item() == 0
    al, be = gdn.gates_from_raw(g.numpy(), b.numpy())
    S, o_ref = gdn.sequential_heads(np.zeros((GH, DV, DK)), bf16.to_f64(bits_of(q)), bf16.to_f64(bits_of(k)),
                                    bf16.to_f64(bits_of(v)), al, be)
    got = pool[1].cpu().numpy().astype(np.float64)
    for h in range(GH):
        rel = np.linalg.norm(got[h] - S[h]) / np.linalg.norm(S[h])
        assert rel <= 1e-4, (h, rel)
    oc = o.cpu().numpy().astype(np.float64)
    for t in list(range(0, N, 997)) + [N - 1]:
        for h in range(GH):
            rel = np.linalg.norm(oc[t, h] - o_ref[t, h]) / max(np.linalg.norm(o_ref[t, h]), 1e-30)
            assert rel <= 1e-4, (t, h, rel)


def test_agentic_turn_resumes_from_the_prefix_cache():
    """A turn of the agentic loop ends: the conversation goes into the radix
    prefix cache (its pages and the GDN checkpoint slot) and the request is
    freed.  The next turn starts from had_radix_match -> had_kvpt_seq_create_from
    on the matched pages and reads the cached checkpoint slot (never writing
    it); its first append copies the shared partial page on the device.
    Attention and the GDN state after the resumed steps must equal the oracle
    run over the whole history."""
    seed, H_q, first, per = 650, 8, 50000, 800
    max_pages = -(-(first + 2 * per + 2) // P) + 1
    N = max_pages + 8
    n_slots = 8
    pt = had.PageTable(N, P, 2, max_pages, free_order=synth.permutation(N, synth.seed_of(seed, 0)))
    slots = had.SlotPool(n_slots, free_order=synth.permutation(n_slots, synth.seed_of(seed, 1)))
    cache = had.RadixCache(pt, slots)
    tokens = synth.integers(0, 49, first + 2 * per + 2, synth.seed_of(seed, 2)).astype(np.int32)
    sq = pt.seq_create()
    pt.reserve(sq, first)
    _say("agentic resume: %d-token first turn + %d steps, cache, %d resumed steps" % (first, per, per))
    kd, vd, kb, vb = _pools(seed, N)
    cur = cur0 = slots.acquire()
    pool0 = np.zeros((n_slots, GH, DV, DK), np.float32)
    pool0[cur] = _warm_state(seed)
    pool_d = to_dev(pool0)
    steps = 2 * per
    qg, k, v, w_q, w_k = _prologue_inputs(seed, steps, 1, H_q)
    gq, gk, gv, gal, gbe = _gdn_inputs(seed, steps, 1)
    qg_d, k_d, v_d, wq_d, wk_d = to_dev(qg), to_dev(k), to_dev(v), to_dev(w_q), to_dev(w_k)
    gdn_d = [to_dev(x) for x in (gq, gk, gv, gal, gbe)]
    table0, _ = pt.export([sq], max_pages)
    first_pages = table0[0, :-(-first // P)].copy()
    lens_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    in_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    out_d = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    src_d = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    dst_d = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    max_len = first + steps + 1
    desc = had.attn_desc((1, 1, H_q, D), kd.shape, max_pages, max_seq_len=max_len, gated=True)
    ws = torch.empty(had.decode_attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    sampled = {}
    first_resumed = []
    n_cow = 0

    def decode(t, seq, L):
        nonlocal cur, n_cow
        out_slot = slots.acquire()
        trip = pt.reserve(seq, 1)
        if trip is not None:                                # the cache shares the partial last page
            src_d.fill_(int(trip[0]))
            dst_d.fill_(int(trip[1]))
            had.kv_copy_pages(kd, vd, src_d, dst_d, d_err=err)
            n_cow += 1
        table, _ = pt.export([seq], max_pages)
        lens_d.fill_(L + 1)
        in_d.fill_(cur)
        out_d.fill_(out_slot)
        out, _ = had.decode_attn_layer(qg_d[t:t + 1], k_d[t:t + 1], v_d[t:t + 1], wq_d, wk_d, to_dev(table), lens_d,
                                       kd, vd, R, max_seq_len=max_len, workspace=ws, d_err=err, gated=True)
        had.gdn_state_update(pool_d, in_d, out_d, *[x[t:t + 1] for x in gdn_d], d_err=err)
        if t in (0, per, per + 1, steps - 1):
            sampled[t] = out.clone()
        if t == per:                                        # the first step read from the cached checkpoint
            first_resumed.append(pool_d[out_slot].clone())
        slots.release(cur)
        cur = out_slot

    for t in range(per):                                    # turn 1
        decode(t, sq, first + t)
    L = first + per
    torch.cuda.synchronize()
    row = pt.export([sq], max_pages)[0][0]
    cache.insert(tokens[:L], row[:-(-L // P)], cur)
    ckpt_slot = cur
    ckpt_bits = pool_d[ckpt_slot].cpu().numpy().copy()
    pt.seq_free(sq)                                         # the request ends; the cache keeps pages + slot
    slots.release(cur)

    m, slot, pages, lock = cache.match(tokens[:L + 1])      # the next turn: the whole history + one token
    assert m == L and slot == ckpt_slot
    sq2 = pt.seq_create_from(pages, m)
    slots.retain(slot)
    cur = slot
    for t in range(per, steps):                             # turn 2, resumed from the cache
        decode(t, sq2, first + t)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert n_cow == 1
    assert np.array_equal(pool_d[ckpt_slot].cpu().numpy(), ckpt_bits)     # the checkpoint was never written

    # oracle: the whole history (prior context, then every decoded row) in fp64
    _, k_rows, v_rows = _oracle_prologue(
        qg.reshape(1, steps, H_q, 2, D), k.reshape(1, steps, H_KV, D), v.reshape(1, steps, H_KV, D), w_q, w_k, 0,
        np.arange(first, first + steps))
    K0, V0 = _context(kb, vb, first_pages, first)
    scale = 1.0 / np.sqrt(D)
    for t, o in sampled.items():
        q_ref, _, _ = _oracle_prologue(qg, k, v, w_q, w_k, t, [first + t])
        ref = A.attention(q_ref, np.concatenate([K0, k_rows[:t + 1]]), np.concatenate([V0, v_rows[:t + 1]]), scale)
        ref = Pr.output_gate(ref, bf16.to_f64(bits_of(qg)[t, :, :, 1]))
        assert_attn_close(o[0], ref)
    f = [_gdn_f64(x)[:, 0] for x in (gq, gk, gv, gal, gbe)]
    # the first resumed step, from the fp32 checkpoint it read: per-step tolerance
    S1, _ = gdn.sequential_heads(ckpt_bits.astype(np.float64), *[x[per:per + 1] for x in f])
    got1 = first_resumed[0].cpu().numpy().astype(np.float64)
    for h in range(GH):
        assert _rel_fro(got1[h], S1[h]) <= 1e-4, h
    # the whole chain in fp64 from the initial state: chain tolerance
    S, _ = gdn.sequential_heads(pool0[cur0].astype(np.float64), *[x[:steps] for x in f])
    got = pool_d[cur].cpu().numpy().astype(np.float64)
    for h in range(GH):
        assert _rel_fro(got[h], S[h]) <= 1e-3, h
    cache.unlock(lock)
    cache.close()
