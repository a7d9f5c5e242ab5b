"""GPU: the allocation-free layer entry point (had_decode_attn_layer_static)
against had_decode_attn_layer with a caller workspace, through the C ABI.

Both run the same kernels with the same split plan; with the deterministic
flag their outputs, gate outputs and written pools must agree bit for bit.
Three calls in a row share the library's one per-GPU array: a 64-row MFMA
layer (the prologue's q goes to the array's q block), then two smaller
8-row VALU layers, so a stale partial or q left by an earlier, larger call
would show."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from gpu_util import DEV, bits_of, paged_case, to_dev

pytestmark = pytest.mark.gpu


def _layer_inputs(seed, L, T, H_q, D, P):
    _, k_pool, v_pool, pt, lens = paged_case(seed, [L], T, H_q, 1, D, P)
    qg = to_dev(synth.normal_bf16((1, T, H_q, 2, D), synth.seed_of(seed, 1)))
    k = to_dev(synth.normal_bf16((1, T, 1, D), synth.seed_of(seed, 2)))
    v = to_dev(synth.normal_bf16((1, T, 1, D), synth.seed_of(seed, 3)))
    w_q = to_dev(synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 4)))
    w_k = to_dev(synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(seed, 5)))
    return qg, k, v, w_q, w_k, to_dev(k_pool), to_dev(v_pool), to_dev(pt), to_dev(lens)


@pytest.mark.parametrize("gated", [False, True])
def test_static_workspace_layer_equals_caller_workspace_layer(gated):
    # (seed, context incl. new tokens, new tokens, query heads, head_dim, page size, rotary dims): larger
    # first; 64 rows with 64 rotary dims run the prologue inside the MFMA partial, with 32 as its own
    # kernel writing q to the workspace's q block
    cases = [(9100, 20000, 4, 16, 256, 64, 64), (9103, 12000, 4, 16, 256, 64, 32), (9101, 9000, 1, 8, 256, 64, 64),
             (9102, 700, 1, 8, 128, 16, 64)]
    for seed, L, T, H_q, D, P, R in cases:
        print("case static workspace: L=%d T=%d H_q=%d D=%d R=%d gated=%d" % (L, T, H_q, D, R, gated), flush=True)
        qg, k, v, w_q, w_k, kd, vd, pt, lens = _layer_inputs(seed, L, T, H_q, D, P)
        kd2, vd2 = kd.clone(), vd.clone()
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        out_a = torch.empty((1, T, H_q, D), dtype=torch.bfloat16, device=DEV)
        gate_a = torch.empty_like(out_a)
        out_b, gate_b = torch.empty_like(out_a), torch.empty_like(out_a)
        # at 16 rows or more q is written only when the caller asks for it
        # (where the prologue runs as its own kernel it goes to the
        # workspace's q block instead): leave q_out unset on the MFMA cases
        mfma = T * H_q >= 16
        q_a = None if mfma else torch.empty_like(out_a)
        q_b = None if mfma else torch.empty_like(out_a)
        had.decode_attn_layer(qg, k, v, w_q, w_k, pt, lens, kd, vd, R, out=out_a, gate_out=gate_a, q_out=q_a,
                              d_err=err, deterministic=True, gated=gated)
        had.decode_attn_layer_static(qg, k, v, w_q, w_k, pt, lens, kd2, vd2, R, out_b, gate_b, q_out=q_b, d_err=err,
                                     deterministic=True, gated=gated)
        torch.cuda.synchronize()
        assert err.item() == 0
        assert np.array_equal(bits_of(out_a), bits_of(out_b))
        assert np.array_equal(bits_of(gate_a), bits_of(gate_b))
        if not mfma:
            assert np.array_equal(bits_of(q_a), bits_of(q_b))
        assert np.array_equal(bits_of(kd), bits_of(kd2), equal_nan=True)
        assert np.array_equal(bits_of(vd), bits_of(vd2), equal_nan=True)


def test_static_workspace_rejects_a_layer_that_does_not_fit():
    # 64 sequences x 8 rows x 256 splits x (256 + 2) floats = 135 MB > 32 MiB
    S, H_q, D, P = 64, 8, 256, 64
    qg = torch.zeros((S, 1, H_q, 2, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((S, 1, 1, D), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(D, dtype=torch.float32, device=DEV)
    pool = torch.zeros((8, 1, P, D), dtype=torch.bfloat16, device=DEV)
    pt = torch.zeros((S, 4), dtype=torch.int32, device=DEV)
    lens = torch.full((S,), 100, dtype=torch.int32, device=DEV)
    out = torch.empty((S, 1, H_q, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(had.HadError) as e:
        had.decode_attn_layer_static(qg, k, k, w, w, pt, lens, pool, pool.clone(), 64, out, torch.empty_like(out),
                                     num_splits=256)
    assert e.value.kind == "workspace_too_small"
