"""Helpers for the GPU parity tests: build paged inputs from the seeded
generators, move them to the device, compare with the oracle."""

import numpy as np
import torch

import synth
from oracle import bf16

DEV = "cuda"


def to_dev(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(DEV).contiguous()


def bits_of(t):
    return synth.bits(t)


def nan_bf16(shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16)


def paged_case(seed, lens, q_len, H_q, H_kv, D, P, extra_pages=3, structured=False, stale_nan=True):
    """Random paged KV cache holding len(lens) sequences.

    Pages are a seeded permutation of the pool; rows past each sequence's
    length (and unused pages) hold NaN when stale_nan, so any leak of stale
    data shows up.  Returns host tensors (bf16) and numpy page table/lens.
    """
    n_seqs = len(lens)
    need = [-(-L // P) for L in lens]
    max_pages = max(need) + 1
    N = sum(need) + extra_pages
    perm = synth.permutation(N, synth.seed_of(seed, 1))
    pt = np.full((n_seqs, max_pages), -1, np.int32)
    k_pool = nan_bf16((N, H_kv, P, D)) if stale_nan else synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 2))
    v_pool = nan_bf16((N, H_kv, P, D)) if stale_nan else synth.normal_bf16((N, H_kv, P, D), synth.seed_of(seed, 3))
    at = 0
    for s, L in enumerate(lens):
        pages = perm[at:at + need[s]]
        at += need[s]
        pt[s, :need[s]] = pages
        kk = synth.normal_bf16((L, H_kv, D), synth.seed_of(seed, 10, s))
        if structured:
            vv = synth.normal_bf16_offset((L, H_kv, D), synth.seed_of(seed, 11, s))
        else:
            vv = synth.normal_bf16((L, H_kv, D), synth.seed_of(seed, 11, s))
        t = torch.arange(L)
        ph = torch.from_numpy(pages.astype(np.int64))[t // P]
        k_pool[ph, :, t % P, :] = kk
        v_pool[ph, :, t % P, :] = vv
    q = synth.normal_bf16((n_seqs, q_len, H_q, D), synth.seed_of(seed, 4), scale=4.0 if structured else 1.0)
    return q, k_pool, v_pool, pt, np.asarray(lens, np.int32)


def assert_attn_close(out, ref, atol=1e-2, rel=1e-2):
    got = bf16.to_f64(bits_of(out))
    assert np.all(np.isfinite(got)), "non-finite attention output"
    err = np.abs(got - ref)
    assert err.max() <= atol, "max abs error %.3g" % err.max()
    num = np.sqrt(np.sum((got - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    worst = np.max(num / np.maximum(den, 1e-30))
    assert worst <= rel, "worst per-row relative L2 error %.3g" % worst
