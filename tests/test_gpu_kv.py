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


def test_copy_rejects_overlapping_lists():
    k = torch.zeros((4, 1, 16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(had.HadError):
        had.kv_copy_pages(k, k.clone(), [0, 1], [1, 2])
