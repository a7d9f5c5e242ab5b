"""GPU: the library's calls captured in a HIP graph and replayed.

Each replay runs after eager work and a synchronisation, with new control
data (sequence lengths, slot indices, token offsets) copied into the
device buffers the graph reads, and is compared bit for bit with the same
calls run eagerly from the same starting state (the attention runs with the
deterministic flag, so its bits depend on the inputs and the split plan
only)."""

import numpy as np
import pytest
import torch

import hybrid_attention_decode_amd as had
import synth
from gpu_util import DEV, bits_of, paged_case, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_layer_pair_replays_equal_eager_runs():
    # one attention layer (fused prologue, gated output) and one GDN layer
    # (raw gates, slot ping-pong) of the agentic shape, 4 replays at growing
    # lengths
    P, H_q, H_kv, D, R = 64, 8, 1, 256, 64
    GH, DK = 8, 128
    L0 = 3000
    _, k_pool, v_pool, pt, _ = paged_case(7000, [L0 + 8], 1, H_q, H_kv, D, P)
    qg = to_dev(synth.normal_bf16((1, 1, H_q, 2, D), synth.seed_of(7000, 1)))
    k = to_dev(synth.normal_bf16((1, 1, H_kv, D), synth.seed_of(7000, 2)))
    v = to_dev(synth.normal_bf16((1, 1, H_kv, D), synth.seed_of(7000, 3)))
    w = to_dev(synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(7000, 4)))
    gq = to_dev(synth.l2_normalised_bf16((1, 1, GH, DK), synth.seed_of(7000, 5)))
    gk = to_dev(synth.l2_normalised_bf16((1, 1, GH, DK), synth.seed_of(7000, 6)))
    gv = to_dev(synth.normal_bf16((1, 1, GH, DK), synth.seed_of(7000, 7)))
    graw = to_dev(-synth.uniform_f32((1, 1, GH), 0.0, 0.1, synth.seed_of(7000, 8)))
    braw = to_dev(synth.uniform_f32((1, 1, GH), -2.0, 2.0, synth.seed_of(7000, 9)))
    pool0 = to_dev(synth.normal_f32((3, GH, DK, DK), synth.seed_of(7000, 10)) * 0.1)
    kd0, vd0 = to_dev(k_pool), to_dev(v_pool)
    ptd = to_dev(pt)
    max_len = L0 + 8

    # graph state: pools and the control block the graph reads
    kd, vd, pool = kd0.clone(), vd0.clone(), pool0.clone()
    lens = torch.tensor([L0], dtype=torch.int32, device=DEV)
    i_in = torch.tensor([0], dtype=torch.int32, device=DEV)
    i_out = torch.tensor([[1]], dtype=torch.int32, device=DEV)
    out = torch.empty((1, 1, H_q, D), dtype=torch.bfloat16, device=DEV)
    gate = torch.empty_like(out)
    o = torch.empty((1, 1, GH, DK), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = had.attn_desc((1, 1, H_q, D), kd.shape, pt.shape[1], max_seq_len=max_len, deterministic=True, gated=True)
    ws = torch.empty(had.decode_attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)

    def layer_pair(kd_, vd_, pool_, lens_, in_, out_idx_, out_, gate_, o_, ws_):
        had.decode_attn_layer(qg, k, v, w, w, ptd, lens_, kd_, vd_, R, max_seq_len=max_len, workspace=ws_, out=out_,
                              gate_out=gate_, d_err=err, deterministic=True, gated=True)
        had.gdn_state_update(pool_, in_, out_idx_, gq, gk, gv, graw, braw, o=o_, d_err=err, raw_gates=True)

    g = _capture(lambda: layer_pair(kd, vd, pool, lens, i_in, i_out, out, gate, o, ws))
    for rep, (L, a, b) in enumerate([(L0 + 1, 0, 1), (L0 + 2, 1, 2), (L0 + 5, 2, 0), (L0 + 8, 0, 2)]):
        print("case graph replay %d: L=%d slots %d->%d" % (rep, L, a, b), flush=True)
        # reset the state eagerly, set the control block, replay
        kd.copy_(kd0)
        vd.copy_(vd0)
        pool.copy_(pool0)
        lens.fill_(L)
        i_in.fill_(a)
        i_out.fill_(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, gate, o, kd, vd, pool)]
        # the same calls eagerly from the same state
        kd2, vd2, pool2 = kd0.clone(), vd0.clone(), pool0.clone()
        out2, gate2, o2 = torch.empty_like(out), torch.empty_like(gate), torch.empty_like(o)
        ws2 = torch.empty_like(ws)
        layer_pair(kd2, vd2, pool2, torch.tensor([L], dtype=torch.int32, device=DEV),
                   torch.tensor([a], dtype=torch.int32, device=DEV), torch.tensor([[b]], dtype=torch.int32, device=DEV),
                   out2, gate2, o2, ws2)
        torch.cuda.synchronize()
        assert err.item() == 0
        for x, y in zip(got, (out2, gate2, o2, kd2, vd2, pool2)):
            assert np.array_equal(bits_of(x), bits_of(y), equal_nan=True)


@pytest.mark.parametrize("n_segments", [0, 3])
def test_gdn_prefill_replays_equal_eager_runs(n_segments):
    # the prefill captured once for a max_len bound, replayed on different
    # packings of the same token buffer (cu_seqlens and slots change); also
    # with the scan in segments (its link reads the input slot, the last
    # segment writes the output slot)
    H, DK, DV, N = 4, 128, 128, 700
    q = to_dev(synth.l2_normalised_bf16((N, H, DK), synth.seed_of(7100, 1)))
    k = to_dev(synth.l2_normalised_bf16((N, H, DK), synth.seed_of(7100, 2)))
    v = to_dev(synth.normal_bf16((N, H, DV), synth.seed_of(7100, 3)))
    al = to_dev(synth.uniform_f32((N, H), 0.9, 1.0, synth.seed_of(7100, 4)))
    be = to_dev(synth.uniform_f32((N, H), 0.0, 1.0, synth.seed_of(7100, 5)))
    pool0 = to_dev(synth.normal_f32((6, H, DV, DK), synth.seed_of(7100, 6)) * 0.1)
    max_len = 400
    cu = torch.zeros(3, dtype=torch.int32, device=DEV)
    i_in = torch.zeros(2, dtype=torch.int32, device=DEV)
    i_out = torch.zeros(2, dtype=torch.int32, device=DEV)
    pool = pool0.clone()
    o = torch.zeros((N, H, DV), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = had.gdn_prefill_desc(pool.shape, 2, max_len, n_segments=n_segments)
    ws = torch.empty(had.gdn_prefill_workspace_bytes(desc), dtype=torch.uint8, device=DEV)

    def run(pool_, cu_, in_, out_, o_, ws_):
        had.gdn_prefill(pool_, in_, out_, cu_, q, k, v, al, be, max_len=max_len, o=o_, workspace=ws_, d_err=err,
                        n_segments=n_segments)

    cu.copy_(torch.tensor([0, 300, 700], dtype=torch.int32))
    i_in.copy_(torch.tensor([0, -1], dtype=torch.int32))
    i_out.copy_(torch.tensor([1, 2], dtype=torch.int32))
    g = _capture(lambda: run(pool, cu, i_in, i_out, o, ws))
    for rep, (c, a, b) in enumerate([([0, 300, 700], [0, -1], [1, 2]), ([0, 64, 464], [3, 3], [4, 5]),
                                     ([0, 0, 1], [-1, 2], [0, 1]), ([0, 399, 700], [5, 4], [5, 3])]):
        print("case prefill replay %d (segments %d): cu=%s in=%s out=%s" % (rep, n_segments, c, a, b), flush=True)
        pool.copy_(pool0)
        o.zero_()
        err.zero_()
        cu.copy_(torch.tensor(c, dtype=torch.int32))
        i_in.copy_(torch.tensor(a, dtype=torch.int32))
        i_out.copy_(torch.tensor(b, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_pool, got_o = pool.clone(), o.clone()
        pool2, o2 = pool0.clone(), torch.zeros_like(o)
        run(pool2, torch.tensor(c, dtype=torch.int32, device=DEV), torch.tensor(a, dtype=torch.int32, device=DEV),
            torch.tensor(b, dtype=torch.int32, device=DEV), o2, torch.empty_like(ws))
        torch.cuda.synchronize()
        assert err.item() == 0
        assert np.array_equal(got_pool.cpu().numpy(), pool2.cpu().numpy())
        n = c[-1]
        assert np.array_equal(got_o[:n].cpu().numpy(), o2[:n].cpu().numpy())


def test_speculative_layer_replays_equal_eager_runs():
    # 16 query heads x 4 drafts per KV head: the MFMA partial with the
    # prologue inside + combine, gated output; 3 replays at different lengths
    P, H_q, H_kv, D, R, T = 64, 16, 1, 256, 64, 4
    L0 = 2500
    _, k_pool, v_pool, pt, _ = paged_case(7100, [L0 + 3 * T], 1, H_q, H_kv, D, P)
    qg = to_dev(synth.normal_bf16((1, T, H_q, 2, D), synth.seed_of(7100, 1)))
    k = to_dev(synth.normal_bf16((1, T, H_kv, D), synth.seed_of(7100, 2)))
    v = to_dev(synth.normal_bf16((1, T, H_kv, D), synth.seed_of(7100, 3)))
    w = to_dev(synth.uniform_f32((D,), 0.5, 1.5, synth.seed_of(7100, 4)))
    kd0, vd0, ptd = to_dev(k_pool), to_dev(v_pool), to_dev(pt)
    max_len = L0 + 3 * T
    kd, vd = kd0.clone(), vd0.clone()
    lens = torch.tensor([L0], dtype=torch.int32, device=DEV)
    out = torch.empty((1, T, H_q, D), dtype=torch.bfloat16, device=DEV)
    gate = torch.empty_like(out)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = had.attn_desc((1, T, H_q, D), kd.shape, pt.shape[1], max_seq_len=max_len, deterministic=True, gated=True)
    ws = torch.empty(had.decode_attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)

    def layer(kd_, vd_, lens_, out_, gate_, ws_):
        had.decode_attn_layer(qg, k, v, w, w, ptd, lens_, kd_, vd_, R, max_seq_len=max_len, workspace=ws_, out=out_,
                              gate_out=gate_, d_err=err, deterministic=True, gated=True)

    g = _capture(lambda: layer(kd, vd, lens, out, gate, ws))
    for rep, L in enumerate([L0 + T, L0 + 2 * T + 1, L0 + 3 * T]):
        print("case speculative graph replay %d: L=%d" % (rep, L), flush=True)
        kd.copy_(kd0)
        vd.copy_(vd0)
        lens.fill_(L)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, gate, kd, vd)]
        kd2, vd2 = kd0.clone(), vd0.clone()
        out2, gate2, ws2 = torch.empty_like(out), torch.empty_like(gate), torch.empty_like(ws)
        layer(kd2, vd2, torch.tensor([L], dtype=torch.int32, device=DEV), out2, gate2, ws2)
        torch.cuda.synchronize()
        assert err.item() == 0
        for x, y in zip(got, (out2, gate2, kd2, vd2)):
            assert np.array_equal(bits_of(x), bits_of(y), equal_nan=True)


def test_cascade_replays_equal_eager_runs():
    # 16 sequences on one 40-page prefix (128 rows in the prefix pass), each
    # with 3 private pages; the suffix lengths change between replays
    n, P, H_q, H_kv, D, pp, priv = 16, 64, 8, 1, 256, 40, 3
    N = pp + n * priv + 2
    order = synth.permutation(N, synth.seed_of(7200, 0))
    table = np.zeros((n, pp + priv + 1), np.int32)
    for s in range(n):
        table[s, :pp] = order[:pp]
        table[s, pp:pp + priv] = order[pp + s * priv:pp + (s + 1) * priv]
        table[s, pp + priv] = order[-1]
    kd = to_dev(synth.normal_bf16((N, H_kv, P, D), synth.seed_of(7200, 1)))
    vd = to_dev(synth.normal_bf16((N, H_kv, P, D), synth.seed_of(7200, 2)))
    q = to_dev(synth.normal_bf16((n, 1, H_q, D), synth.seed_of(7200, 3)))
    gt = to_dev(synth.normal_bf16((n, 1, H_q, D), synth.seed_of(7200, 4)))
    ptd, prefix = to_dev(table), to_dev(table[0, :pp].copy())
    max_len = (pp + priv) * P
    lens = torch.zeros(n, dtype=torch.int32, device=DEV)
    out = torch.empty((n, 1, H_q, D), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = had.attn_desc(q.shape, kd.shape, table.shape[1], max_seq_len=max_len, deterministic=True, gated=True)
    ws = torch.empty(had.decode_attn_cascade_workspace_bytes(desc, pp), dtype=torch.uint8, device=DEV)

    def run(lens_, out_, ws_):
        had.decode_attn_cascade(q, kd, vd, ptd, lens_, prefix, max_seq_len=max_len, workspace=ws_, out=out_,
                                d_err=err, deterministic=True, gate=gt)

    lens.copy_(torch.from_numpy(np.full(n, pp * P + 1, np.int32)))
    g = _capture(lambda: run(lens, out, ws))
    for rep in range(3):
        L = pp * P + synth.integers(1, priv * P + 1, n, synth.seed_of(7200, 10 + rep))
        print("case cascade graph replay %d: lens=%s" % (rep, [int(x) for x in L]), flush=True)
        lens.copy_(torch.from_numpy(L.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out2, ws2 = torch.empty_like(out), torch.empty_like(ws)
        run(to_dev(L.astype(np.int32)), out2, ws2)
        torch.cuda.synchronize()
        assert err.item() == 0
        assert np.array_equal(bits_of(got), bits_of(out2), equal_nan=True)
