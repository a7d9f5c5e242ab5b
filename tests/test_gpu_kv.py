"""GPU parity: KV append and copy-on-write page copies, bit for bit."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from oracle import paging
from gpu_util import DEV, bits_of, to_dev

pytestmark = pytest.mark.gpu


def test_append_writes_the_addressed_page_rows():
    N, H_kv, P, D = 12, 2, 16, 64
    k_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(1, 1))
    v_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(1, 2))
    pt = np.array([[5, 2, 9, -1], [7, 0, -1, -1]], np.int32)
    lens = np.array([40, 20], np.int32)
    t_new = 3
    k_new = synth.normal_bf16((2, t_new, H_kv, D), synth.seed_of(1, 3))
    v_new = synth.normal_bf16((2, t_new, H_kv, D), synth.seed_of(1, 4))
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    had.kv_append(kd, vd, to_dev(pt), to_dev(lens), to_dev(k_new), to_dev(v_new))
    torch.cuda.synchronize()
    exp_k, exp_v = bits_of(k_pool).copy(), bits_of(v_pool).copy()
    for s in range(2):
        for j in range(t_new):
            pos = lens[s] - t_new + j
            exp_k[pt[s, pos // P], :, pos % P] = bits_of(k_new)[s, j]
            exp_v[pt[s, pos // P], :, pos % P] = bits_of(v_new)[s, j]
    assert np.array_equal(bits_of(kd), exp_k) and np.array_equal(bits_of(vd), exp_v)


def test_copy_on_write_after_fork():
    P, N, H_kv, D = 16, 10, 1, 128
    pt = had.PageTable(N, P, 4, 8, free_order=synth.permutation(N, 5))
    a = pt.seq_create()
    assert pt.reserve(a, 40) is None
    k_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(2, 1))
    v_pool = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(2, 2))
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    b = pt.seq_fork(a, 40)
    cow = pt.reserve(b, 1)
    assert cow is not None and cow[2] == 40 % P
    src, dst, valid = cow
    had.kv_copy_pages(kd, vd, [src], [dst])
    torch.cuda.synchronize()
    kb, vb = bits_of(kd), bits_of(vd)
    assert np.array_equal(kb[src], bits_of(k_pool)[src])            # source untouched
    assert np.array_equal(kb[dst, :, :valid], kb[src, :, :valid])   # valid rows copied
    assert np.array_equal(vb[dst, :, :valid], vb[src, :, :valid])
    others = [p for p in range(N) if p != dst]
    assert np.array_equal(kb[others], bits_of(k_pool)[others])
    tab, lens = pt.export([a, b], 8)
    ga = paging.gather(kb, tab[0], 40, P)
    gb = paging.gather(kb, tab[1], 40, P)
    assert np.array_equal(ga, gb)                                    # same logical prefix


def test_copy_list_errors_are_reported_on_the_device():
    # pairs live in device memory: a bad pair is skipped and reported, the
    # others are copied, and -1 entries do nothing
    N, P, D = 12, 16, 64
    k0 = synth.normal_bf16((N, 1, P, D), synth.seed_of(3, 1))
    v0 = synth.normal_bf16((N, 1, P, D), synth.seed_of(3, 2))
    cases = [
        # (src, dst, error bits, pairs that must have been copied)
        ([2, -1, 5], [7, 3, 8], 0, [(2, 7), (5, 8)]),
        ([2, 4], [4, 9], had.DERR_COPY, [(4, 9)]),          # 4 is a source: pair 0 races, skipped
        ([2, 3], [9, 9], had.DERR_COPY, [(2, 9)]),          # repeated destination: the later pair skipped
        ([2, 30], [6, 7], had.DERR_PAGE, [(2, 6)]),         # source out of range
        ([-3], [6], had.DERR_PAGE, []),                     # only -1 marks an unused entry
    ]
    for src, dst, bits, copied in cases:
        print("case copy list %s -> %s" % (src, dst), flush=True)
        kd, vd = to_dev(k0), to_dev(v0)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        had.kv_copy_pages(kd, vd, to_dev(np.array(src, np.int32)), to_dev(np.array(dst, np.int32)), d_err=err)
        torch.cuda.synchronize()
        assert err.item() == bits
        exp_k, exp_v = bits_of(k0).copy(), bits_of(v0).copy()
        for a, b in copied:
            exp_k[b], exp_v[b] = exp_k[a], exp_v[a]
        assert np.array_equal(bits_of(kd), exp_k) and np.array_equal(bits_of(vd), exp_v)
    with pytest.raises(had.HadError):                      # the same checks on the host
        had.kv_check_copy_pages(N, [2, 4], [4, 9])


def test_copy_on_write_inside_a_replayed_graph():
    # a captured step holds the page copy and a raw append; the host manager
    # (C++) and the oracle's page-table model run the same forks and appends,
    # each replay gets the step's copy pairs (unused entries -1) and the new
    # lengths through device buffers, and the pools must equal the oracle's
    # pools bit for bit after every replay
    N, P, H_kv, D, S = 24, 16, 1, 64, 3
    max_pages = 8
    order = synth.permutation(N, synth.seed_of(4, 0))
    pt = had.PageTable(N, P, S + 1, max_pages, free_order=order)
    model = paging.PageTableModel(N, P, S + 1, max_pages, free_order=order)
    k0 = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(4, 1))
    v0 = synth.normal_bf16((N, H_kv, P, D), synth.seed_of(4, 2))
    kd, vd = to_dev(k0), to_dev(v0)
    kb, vb = bits_of(k0).copy(), bits_of(v0).copy()
    root, mroot = pt.seq_create(), model.seq_create()
    pt.reserve(root, 37)
    model.reserve(mroot, 37)
    seqs = [pt.seq_fork(root, 37) for _ in range(S)]
    mseqs = [model.seq_fork(mroot, 37) for _ in range(S)]

    src_d = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    dst_d = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    pt_d = torch.full((S, max_pages), -1, dtype=torch.int32, device=DEV)
    lens_d = torch.zeros(S, dtype=torch.int32, device=DEV)
    k_new = torch.empty((S, 1, H_kv, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        had.kv_copy_pages(kd, vd, src_d, dst_d, d_err=err)
        had.kv_append(kd, vd, pt_d, lens_d, k_new, v_new, d_err=err)

    # capture only (nothing runs until the first replay)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    who = [[0, 1, 2], [1], [0, 2], [2, 0, 1]]            # sequences that append a token, per replay
    for rep, active in enumerate(who):
        src = np.full(S, -1, np.int32)
        dst = np.full(S, -1, np.int32)
        lens_h = np.zeros(S, np.int32)
        for i in active:
            trip, mtrip = pt.reserve(seqs[i], 1), model.reserve(mseqs[i], 1)
            assert (trip is None) == (mtrip is None)
            if mtrip is not None:
                assert tuple(trip) == tuple(mtrip)
                src[i], dst[i] = mtrip[0], mtrip[1]
                kb[mtrip[1]], vb[mtrip[1]] = kb[mtrip[0]], vb[mtrip[0]]
        table, lens = pt.export(seqs, max_pages)
        mtable, mlens = model.export(mseqs, max_pages)
        assert np.array_equal(table, mtable) and np.array_equal(lens, mlens)
        # sequences not appending this replay point at no row (length 0 -> SEQLEN would fire), so
        # the append runs for the active ones only: inactive rows get a length whose row is
        # rewritten with the bytes it already holds
        knew = synth.normal_bf16((S, 1, H_kv, D), synth.seed_of(4, 10, rep))
        vnew = synth.normal_bf16((S, 1, H_kv, D), synth.seed_of(4, 11, rep))
        for i in range(S):
            L = int(lens[i])
            page, row = mtable[i][(L - 1) // P], (L - 1) % P
            if i in active:
                kb[page, :, row], vb[page, :, row] = bits_of(knew)[i, 0], bits_of(vnew)[i, 0]
            else:
                knew[i, 0] = torch.from_numpy(np.ascontiguousarray(kb[page, :, row]).view(np.int16)).view(torch.bfloat16)
                vnew[i, 0] = torch.from_numpy(np.ascontiguousarray(vb[page, :, row]).view(np.int16)).view(torch.bfloat16)
            lens_h[i] = L
        print("case graph CoW replay %d: pairs %s -> %s" % (rep, list(src), list(dst)), flush=True)
        src_d.copy_(torch.from_numpy(src))
        dst_d.copy_(torch.from_numpy(dst))
        pt_d.copy_(torch.from_numpy(table))
        lens_d.copy_(torch.from_numpy(lens_h))
        k_new.copy_(knew)
        v_new.copy_(vnew)
        g.replay()
        torch.cuda.synchronize()
        assert err.item() == 0
        assert np.array_equal(bits_of(kd), kb) and np.array_equal(bits_of(vd), vb), rep
    # every sequence now reads the shared prefix rows through its own pages
    table, lens = pt.export(seqs, max_pages)
    kb_now = bits_of(kd)
    ref = paging.gather(kb_now, table[0], 37, P)
    for i in range(1, S):
        assert np.array_equal(paging.gather(kb_now, table[i], 37, P), ref)
