#!/usr/bin/env python3
"""Decode-step benchmark of the hybrid-attention decode path on one MI355X.

Workload (long-context sweep): one sequence decoding at contexts 128K, 256K
and 1M tokens through a 48-layer hybrid stack -- 12 full-attention layers
(8 query heads / 1 KV head, head_dim 256, partial RoPE on 64 dims, bf16 KV in
64-token pages drawn from a randomly permuted pool) and 36 Gated DeltaNet
layers (8 heads, d_k = d_v = 128, fp32 state), layers 4i..4i+2 GDN and 4i+3
attention.  Synthetic seeded inputs; values do not affect timing.

One step = one decode token through the whole stack:
  host   C++ page-table reserve of the new token (+ pinned async H2D of the
         length and, on a page boundary, of the new page-table entry)
  device replay of a captured HIP graph of the 48 layers:
         GDN layer       had_gdn_state_update  (slot ping-pong by index;
                         alpha = exp(g), beta = sigmoid(b) formed in-kernel
                         from the raw gate values)
         attention layer had_decode_attn_layer: the prologue (QK-RMSNorm,
                         partial RoPE, gate split, K/V append) runs inside the
                         split-K partial kernel, then the combine kernel, which
                         applies the output gate sigmoid(gate)
  Every kernel ORs its error bits into one device word, read once after the
  timed region (no per-step device-to-host round trip).

Prints one JSON line (stdout).  Progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s + achieved HBM GB/s (% of peak) at 128K/256K/1M ctx, 1 GPU"
PEAK_HBM_GBPS = 8000.0
P, H_Q, H_KV, D, R = 64, 8, 1, 256, 64
N_ATTN, N_GDN = 12, 36
GDN_H, DK, DV = 8, 128, 128
KV_BYTES_PER_TOKEN = 2 * H_KV * D * 2          # K and V rows, bf16
GDN_BYTES_PER_LAYER = 2 * GDN_H * DK * DV * 4  # state read + write, fp32
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_valu_d256_longctx_pmc.json")
KERNEL_DIR = os.path.join(ROOT, "hybrid_attention_decode_amd", "csrc", "kernels")
# the partial kernel's source and the headers it includes: the PMC summary is
# used only while they are unchanged
KERNEL_SRCS = [os.path.join(KERNEL_DIR, f)
               for f in ("attn_valu.hip", "attn_valu_body.h", "attn_internal.h", "prologue_math.h", "kcommon.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for fn in KERNEL_SRCS:
        with open(fn, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def check_sentinel(st):
    """The one device-to-host read of the run's error word, after timing."""
    e = int(st.err.item())
    if e:
        raise RuntimeError("a kernel reported error bits 0x%x during the run" % e)


def algorithmic_bytes_per_step(L):
    return N_ATTN * L * KV_BYTES_PER_TOKEN + N_GDN * GDN_BYTES_PER_LAYER


class LongContextStack:
    """Device state of the 48-layer stack for one sequence at context L0."""

    def __init__(self, L0, n_tokens, seed=0):
        import torch

        import hybrid_attention_decode_amd as had
        import synth

        self.torch, self.had = torch, had
        dev = "cuda"
        self.L0 = L0
        self.total = L0 + n_tokens
        self.max_pages = -(-self.total // P) + 1
        self.num_pages = self.max_pages + 4
        order = synth.permutation(self.num_pages, synth.seed_of(seed, 1))
        self.pt = had.PageTable(self.num_pages, P, 1, self.max_pages, free_order=order)
        self.seq = self.pt.seq_create()
        self.pt.reserve(self.seq, L0)
        table, lens = self.pt.export([self.seq], self.max_pages)
        self.pt_dev = torch.from_numpy(table).to(dev)
        self.lens_dev = torch.from_numpy(lens).to(dev)
        self.len = L0
        # pinned staging, one entry per step so no buffer is rewritten while a copy is pending
        self.lens_pin = torch.empty(n_tokens + 1, dtype=torch.int32, pin_memory=True)
        # device sentinel: every kernel ORs its error bits here; read once after the run
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.page_pin = torch.empty(n_tokens + 1, dtype=torch.int32, pin_memory=True)

        g = torch.Generator(device=dev)
        self.attn = []
        for i in range(N_ATTN):
            g.manual_seed(synth.seed_of(seed, 100, i))
            lay = dict(
                k_pool=torch.randn((self.num_pages, H_KV, P, D), generator=g, device=dev, dtype=torch.bfloat16),
                v_pool=torch.randn((self.num_pages, H_KV, P, D), generator=g, device=dev, dtype=torch.bfloat16),
                qg=torch.randn((1, 1, H_Q, 2, D), generator=g, device=dev, dtype=torch.bfloat16),
                k=torch.randn((1, 1, H_KV, D), generator=g, device=dev, dtype=torch.bfloat16),
                v=torch.randn((1, 1, H_KV, D), generator=g, device=dev, dtype=torch.bfloat16),
                w_q=torch.rand((D,), generator=g, device=dev) + 0.5,
                w_k=torch.rand((D,), generator=g, device=dev) + 0.5,
                q_out=torch.empty((1, 1, H_Q, D), device=dev, dtype=torch.bfloat16),
                gate=torch.empty((1, 1, H_Q, D), device=dev, dtype=torch.bfloat16),
                out=torch.empty((1, 1, H_Q, D), device=dev, dtype=torch.bfloat16),
            )
            self.attn.append(lay)
        self.desc = had.attn_desc((1, 1, H_Q, D), (self.num_pages, H_KV, P, D), self.max_pages,
                                  max_seq_len=self.total)
        self.n_splits, self.pps = had.decode_attn_plan(self.desc)
        self.ws = torch.empty(had.decode_attn_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        self.gdn = []
        for i in range(N_GDN):
            g.manual_seed(synth.seed_of(seed, 200, i))
            q = torch.randn((1, 1, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
            k = torch.randn((1, 1, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
            lay = dict(
                pool=torch.randn((2, GDN_H, DV, DK), generator=g, device=dev) * 0.05,
                q=(q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16),
                k=(k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16),
                v=torch.randn((1, 1, GDN_H, DV), generator=g, device=dev, dtype=torch.bfloat16),
                g=-0.1 * torch.rand((1, 1, GDN_H), generator=g, device=dev),   # raw log decay
                b=torch.randn((1, 1, GDN_H), generator=g, device=dev),           # raw write strength
                o=torch.empty((1, 1, GDN_H, DV), device=dev),
            )
            self.gdn.append(lay)
        # slot ping-pong by index: even steps read slot 0 and write slot 1, odd steps the reverse
        self.in_idx = [torch.tensor([0], dtype=torch.int32, device=dev), torch.tensor([1], dtype=torch.int32, device=dev)]
        self.out_idx = [torch.tensor([[1]], dtype=torch.int32, device=dev), torch.tensor([[0]], dtype=torch.int32, device=dev)]
        self.graphs = None

    # --- the per-layer calls ---------------------------------------------------
    def attn_layer(self, i):
        a = self.attn[i]
        self.had.decode_attn_layer(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], self.pt_dev, self.lens_dev,
                                   a["k_pool"], a["v_pool"], R, max_seq_len=self.total, workspace=self.ws,
                                   out=a["out"], gate_out=a["gate"], d_err=self.err, gated=True)

    def gdn_layer(self, i, parity):
        g = self.gdn[i]
        self.had.gdn_state_update(g["pool"], self.in_idx[parity], self.out_idx[parity], g["q"], g["k"], g["v"],
                                  g["g"], g["b"], o=g["o"], d_err=self.err, raw_gates=True)

    def layers(self, parity):
        ia = ig = 0
        for l in range(N_ATTN + N_GDN):
            if l % 4 == 3:
                self.attn_layer(ia)
                ia += 1
            else:
                self.gdn_layer(ig, parity)
                ig += 1

    def capture(self):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.layers(0)
            self.layers(1)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graphs = []
        for par in (0, 1):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                self.layers(par)
            self.graphs.append(gr)
        torch.cuda.synchronize()

    # --- one decode step ---------------------------------------------------------
    def step(self, t):
        cow = self.pt.reserve(self.seq, 1)            # host: C++ page-table manager
        assert cow is None                            # one unshared sequence: never copies
        self.len += 1
        pos = self.len - 1
        if pos % P == 0:                              # a new page was allocated for this token
            table, _ = self.pt.export([self.seq], self.max_pages)
            self.page_pin[t] = int(table[0, pos // P])
            self.pt_dev[0, pos // P].copy_(self.page_pin[t], non_blocking=True)
        self.lens_pin[t] = self.len
        self.lens_dev.copy_(self.lens_pin[t:t + 1], non_blocking=True)
        self.graphs[t % 2].replay()


def time_graph(torch, fn, reps, n_timed=5):
    """Average duration of one call of fn, from a captured batch of `reps`
    calls: the median over `n_timed` timed replays of the batch's average."""
    gr = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        for r in range(reps):
            fn(r)
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    batch_ms = []
    for _ in range(n_timed):
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        batch_ms.append(e0.elapsed_time(e1))
    return float(np.median(batch_ms)) * 1e3 / reps  # microseconds


def run_context(L0, steps, warmup, kernel_reps, seed=0):
    import torch

    import hybrid_attention_decode_amd as had

    t0 = time.time()
    st = LongContextStack(L0, steps + warmup + 2, seed)
    st.capture()
    log("ctx %d: setup %.1fs (splits=%d, pages/split=%d)" % (L0, time.time() - t0, st.n_splits, st.pps))
    for t in range(warmup):
        st.step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    len_start = st.len
    e0.record()
    for t in range(warmup, warmup + steps):
        st.step(t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same 48-layer graph replayed back to back without the host-side
    # bookkeeping and copies (device time of a step)
    e0.record()
    for t in range(steps):
        st.graphs[t % 2].replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    mean_len = len_start + (steps + 1) / 2.0
    step_bytes = algorithmic_bytes_per_step(mean_len)
    log("ctx %d: %.4f ms/step, %.1f steps/s" % (L0, ms, 1e3 / ms))

    # per kernel class, captured back-to-back batches rotating over the layers
    L = st.len
    ws = st.ws
    n = max(1, kernel_reps)

    def partial(r):  # the fused kernel: prologue + split-K partials
        a = st.attn[r % N_ATTN]
        had.decode_attn_layer(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], st.pt_dev, st.lens_dev, a["k_pool"],
                              a["v_pool"], R, max_seq_len=st.total, workspace=ws, gate_out=a["gate"],
                              out=a["out"], partial_only=True)

    def combine(r):
        had.decode_attn_combine(st.desc, st.n_splits, ws, st.attn[r % N_ATTN]["out"])

    def gdn(r):
        st.gdn_layer(r % N_GDN, r % 2)

    us = {
        "attn_partial": time_graph(torch, partial, n * N_ATTN),
        "attn_combine": time_graph(torch, combine, n * N_ATTN),
        "gdn_update": time_graph(torch, gdn, max(2, n) * N_GDN),
    }
    attn_bytes = L * KV_BYTES_PER_TOKEN
    res = dict(
        context=L0, steps=steps, warmup=warmup, ms_per_step=ms, steps_per_s=1e3 / ms, graph_only_ms_per_step=graph_ms,
        mean_context_timed=mean_len, algorithmic_bytes_per_step=step_bytes,
        hbm_gbps=step_bytes / (ms * 1e-3) / 1e9, hbm_frac=step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        us_per_layer={k: round(v, 3) for k, v in us.items()},
        attn_us_per_layer=round(us["attn_partial"] + us["attn_combine"], 3),
        attn_partial_gbps=attn_bytes / (us["attn_partial"] * 1e-6) / 1e9,
        attn_partial_bytes_per_launch=attn_bytes, attn_partial_context=L,
        num_splits=st.n_splits, pages_per_split=st.pps,
    )
    check_sentinel(st)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


class Stack:
    """The 48-layer hybrid stack for n_seqs sequences with T new tokens per step.

    Per-step control (sequence lengths, GDN input slot per sequence, GDN output
    slot per (sequence, token)) lives in one device int32 block that the host
    refreshes with a single pinned async copy before each graph replay; the
    page table is patched entry by entry when the host manager hands out a
    new page.
    """

    def __init__(self, n_seqs, T, H_q, num_pages, max_pages, max_seq_len, n_slots, n_steps, seed):
        import torch

        import hybrid_attention_decode_amd as had
        import synth

        self.torch, self.had = torch, had
        dev = "cuda"
        self.n, self.T, self.H_q = n_seqs, T, H_q
        self.num_pages, self.max_pages, self.max_seq_len = num_pages, max_pages, max_seq_len
        n = n_seqs
        # control block: lengths, GDN input slots, GDN output slots, then the
        # copy-on-write pairs (source, destination) per sequence (-1: none)
        self.ctrl_len = 2 * n + n * T + 2 * n
        self.ctrl = torch.zeros(self.ctrl_len, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)  # device sentinel, read after the run
        self.lens_dev = self.ctrl[:n]
        self.in_dev = self.ctrl[n:2 * n]
        self.out_dev = self.ctrl[2 * n:2 * n + n * T].view(n, T)
        self.cow_src = self.ctrl[2 * n + n * T:3 * n + n * T]
        self.cow_dst = self.ctrl[3 * n + n * T:]
        self.ctrl_pin = torch.empty((n_steps + 4, self.ctrl_len), dtype=torch.int32, pin_memory=True)
        self.pt_dev = torch.full((n, max_pages), -1, dtype=torch.int32, device=dev)
        self.pt_pin = torch.empty(n_steps * n * (T // P + 2) + 16, dtype=torch.int32, pin_memory=True)
        self.pt_pin_at = 0
        g = torch.Generator(device=dev)
        self.attn = []
        for i in range(N_ATTN):
            g.manual_seed(synth.seed_of(seed, 100, i))
            self.attn.append(dict(
                k_pool=torch.randn((num_pages, H_KV, P, D), generator=g, device=dev, dtype=torch.bfloat16),
                v_pool=torch.randn((num_pages, H_KV, P, D), generator=g, device=dev, dtype=torch.bfloat16),
                qg=torch.randn((n, T, H_q, 2, D), generator=g, device=dev, dtype=torch.bfloat16),
                k=torch.randn((n, T, H_KV, D), generator=g, device=dev, dtype=torch.bfloat16),
                v=torch.randn((n, T, H_KV, D), generator=g, device=dev, dtype=torch.bfloat16),
                w_q=torch.rand((D,), generator=g, device=dev) + 0.5,
                w_k=torch.rand((D,), generator=g, device=dev) + 0.5,
                q_out=torch.empty((n, T, H_q, D), device=dev, dtype=torch.bfloat16),
                gate=torch.empty((n, T, H_q, D), device=dev, dtype=torch.bfloat16),
                out=torch.empty((n, T, H_q, D), device=dev, dtype=torch.bfloat16)))
        self.desc = had.attn_desc((n, T, H_q, D), (num_pages, H_KV, P, D), max_pages, max_seq_len=max_seq_len)
        self.n_splits, self.pps = had.decode_attn_plan(self.desc)
        self.ws = torch.empty(had.decode_attn_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        self.gdn = []
        for i in range(N_GDN):
            g.manual_seed(synth.seed_of(seed, 200, i))
            q = torch.randn((n, T, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
            k = torch.randn((n, T, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
            self.gdn.append(dict(
                pool=torch.randn((n_slots, GDN_H, DV, DK), generator=g, device=dev) * 0.05,
                q=(q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16),
                k=(k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16),
                v=torch.randn((n, T, GDN_H, DV), generator=g, device=dev, dtype=torch.bfloat16),
                g=-0.1 * torch.rand((n, T, GDN_H), generator=g, device=dev),
                b=torch.randn((n, T, GDN_H), generator=g, device=dev),
                o=torch.empty((n, T, GDN_H, DV), device=dev)))
        self.graph = None

    def enable_cascade(self, prefix_pages_dev):
        """Attention layers read the batch's shared prefix pages once for all
        sequences (had_decode_attn_cascade) after a separate prologue."""
        import torch

        self.prefix_dev = prefix_pages_dev
        nbytes = self.had.decode_attn_cascade_workspace_bytes(self.desc, prefix_pages_dev.numel())
        self.cws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def attn_layer(self, i):
        a = self.attn[i]
        if getattr(self, "prefix_dev", None) is not None:
            self.had.qk_norm_rope_gate(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], self.pt_dev, self.lens_dev,
                                       a["k_pool"], a["v_pool"], R, q_out=a["q_out"], gate_out=a["gate"],
                                       d_err=self.err)
            self.had.decode_attn_cascade(a["q_out"], a["k_pool"], a["v_pool"], self.pt_dev, self.lens_dev,
                                         self.prefix_dev, max_seq_len=self.max_seq_len, workspace=self.cws,
                                         out=a["out"], d_err=self.err, gate=a["gate"])
            return
        self.had.decode_attn_layer(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], self.pt_dev, self.lens_dev,
                                   a["k_pool"], a["v_pool"], R, max_seq_len=self.max_seq_len, workspace=self.ws,
                                   out=a["out"], gate_out=a["gate"], d_err=self.err, gated=True)

    def gdn_layer(self, i):
        g = self.gdn[i]
        self.had.gdn_state_update(g["pool"], self.in_dev, self.out_dev, g["q"], g["k"], g["v"], g["g"], g["b"],
                                  o=g["o"], d_err=self.err, raw_gates=True)

    def layers(self):
        ia = ig = 0
        for l in range(N_ATTN + N_GDN):
            if l % 4 == 3:
                self.attn_layer(ia)
                ia += 1
            else:
                self.gdn_layer(ig)
                ig += 1

    def cow_copies(self):
        """The device half of copy-on-write in every attention layer's pools:
        pairs from the control block (unused entries -1 copy nothing)."""
        for a in self.attn:
            self.had.kv_copy_pages(a["k_pool"], a["v_pool"], self.cow_src, self.cow_dst, d_err=self.err)

    def capture(self):
        """Two step graphs: the 48 layers, and the same step preceded by the
        copy-on-write page copies (replayed on steps whose reservation copied a
        shared partial page)."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.layers()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.layers()
        self.graph_cow = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph_cow):
            self.cow_copies()
            self.layers()
        torch.cuda.synchronize()

    def replay(self, cow):
        (self.graph_cow if cow else self.graph).replay()

    def set_page(self, s, idx, pid):
        """Patch one device page-table entry (pinned staging, never reused)."""
        self.pt_pin[self.pt_pin_at] = int(pid)
        self.pt_dev[s, idx].copy_(self.pt_pin[self.pt_pin_at], non_blocking=True)
        self.pt_pin_at += 1

    def push_ctrl(self, t, lens, in_idx, out_idx, cow=None):
        """cow: per sequence a (source, destination) page pair or None."""
        row = self.ctrl_pin[t]
        n, T = self.n, self.T
        row[:n] = torch_int(lens)
        row[n:2 * n] = torch_int(in_idx)
        row[2 * n:2 * n + n * T] = torch_int(out_idx).reshape(-1)
        src = [-1] * n
        dst = [-1] * n
        for i, c in enumerate(cow or []):
            if c is not None:
                src[i], dst[i] = int(c[0]), int(c[1])
        row[2 * n + n * T:3 * n + n * T] = torch_int(src)
        row[3 * n + n * T:] = torch_int(dst)
        self.ctrl.copy_(row, non_blocking=True)


def torch_int(x):
    import torch

    return torch.as_tensor(np.asarray(x, dtype=np.int32).reshape(-1))


def stack_kernel_us(st, kernel_reps):
    """Per-kernel-class averages from captured back-to-back batches."""
    import torch

    had = st.had
    n = max(1, kernel_reps)

    def partial(r):  # the fused kernel: prologue + split-K partials
        a = st.attn[r % N_ATTN]
        had.decode_attn_layer(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], st.pt_dev, st.lens_dev, a["k_pool"],
                              a["v_pool"], R, max_seq_len=st.max_seq_len, workspace=st.ws, gate_out=a["gate"],
                              out=a["out"], partial_only=True)

    def combine(r):
        had.decode_attn_combine(st.desc, st.n_splits, st.ws, st.attn[r % N_ATTN]["out"])

    def gdn(r):
        st.gdn_layer(r % N_GDN)

    if getattr(st, "prefix_dev", None) is not None:
        def prologue(r):
            a = st.attn[r % N_ATTN]
            had.qk_norm_rope_gate(a["qg"], a["k"], a["v"], a["w_q"], a["w_k"], st.pt_dev, st.lens_dev, a["k_pool"],
                                  a["v_pool"], R, q_out=a["q_out"], gate_out=a["gate"])

        def cascade(r):
            a = st.attn[r % N_ATTN]
            had.decode_attn_cascade(a["q_out"], a["k_pool"], a["v_pool"], st.pt_dev, st.lens_dev, st.prefix_dev,
                                    max_seq_len=st.max_seq_len, workspace=st.cws, out=a["out"], gate=a["gate"])

        ns_p, ns_s = had.decode_attn_cascade_plan(st.desc, st.prefix_dev.numel())

        def prefix_pass(r):
            a = st.attn[r % N_ATTN]
            had.decode_attn_cascade_partial(a["q_out"], a["k_pool"], a["v_pool"], st.pt_dev, st.lens_dev,
                                            st.prefix_dev, st.cws, 1, max_seq_len=st.max_seq_len)

        def suffix_pass(r):
            a = st.attn[r % N_ATTN]
            had.decode_attn_cascade_partial(a["q_out"], a["k_pool"], a["v_pool"], st.pt_dev, st.lens_dev,
                                            st.prefix_dev, st.cws, 2, max_seq_len=st.max_seq_len)

        def merge(r):
            a = st.attn[r % N_ATTN]
            had.decode_attn_cascade_combine(a["q_out"], a["k_pool"], a["v_pool"], st.pt_dev, st.lens_dev,
                                            st.prefix_dev, st.cws, out=a["out"], max_seq_len=st.max_seq_len,
                                            gate=a["gate"])

        # the whole call (both passes in one launch, then the merge), and the
        # two-pass form through the split entry points, pass by pass
        return {
            "prologue": round(time_graph(torch, prologue, n * N_ATTN), 3),
            "attn_cascade_one_launch_and_merge": round(time_graph(torch, cascade, n * N_ATTN), 3),
            "two_pass_prefix_pass": round(time_graph(torch, prefix_pass, n * N_ATTN), 3),
            "two_pass_suffix_pass": round(time_graph(torch, suffix_pass, n * N_ATTN), 3),
            "two_pass_merge": round(time_graph(torch, merge, n * N_ATTN), 3),
            "two_pass_splits": [ns_p, ns_s],
            "gdn_update": round(time_graph(torch, gdn, max(2, n) * N_GDN), 3),
        }
    return {
        "attn_partial": round(time_graph(torch, partial, n * N_ATTN), 3),
        "attn_combine": round(time_graph(torch, combine, n * N_ATTN), 3),
        "gdn_update": round(time_graph(torch, gdn, max(2, n) * N_GDN), 3),
    }


def run_speculative(L0=262144, steps=256, warmup=10, kernel_reps=4, T=4, G=16, seed=5):
    """Speculative verify: T drafts per step, GQA group G (G*T query rows per KV
    head, MFMA path), GDN checkpoint per draft token into fresh slots, accepted
    length ~ U{0..T} (seeded), rollback by index."""
    import torch

    import hybrid_attention_decode_amd as had
    import synth

    n_steps = steps + warmup
    max_len = L0 + (n_steps + 2) * T
    max_pages = -(-max_len // P) + 1
    num_pages = max_pages + 8
    n_slots = 2 * T + 2
    st = Stack(1, T, G, num_pages, max_pages, max_len, n_slots, n_steps, seed)
    pt = had.PageTable(num_pages, P, 1, max_pages, free_order=synth.permutation(num_pages, synth.seed_of(seed, 1)))
    slots = had.SlotPool(n_slots, free_order=synth.permutation(n_slots, synth.seed_of(seed, 2)))
    seq = pt.seq_create()
    pt.reserve(seq, L0)
    table, _ = pt.export([seq], max_pages)
    st.pt_dev.copy_(torch.from_numpy(table))
    cur = slots.acquire()
    accepted = synth.integers(0, T, n_steps, synth.seed_of(seed, 3))
    L = L0

    def step(t):
        nonlocal cur, L
        outs = [slots.acquire() for _ in range(T)]
        held = -(-L // P)
        assert pt.reserve(seq, T) is None
        if -(-(L + T) // P) > held:                    # pages handed out for the drafts
            row = pt.export([seq], max_pages)[0][0]
            for idx in range(held, -(-(L + T) // P)):
                st.set_page(0, idx, row[idx])
        st.push_ctrl(t, [L + T], [cur], [outs])
        st.replay(False)
        a = int(accepted[t])
        cur = had.spec_rollback(pt, slots, seq, T, a, cur, outs)
        L += a

    # the capture's eager run: the last T held positions stand in for drafts
    # (every page it reads is mapped), checkpoints into distinct free slots
    tmp = [slots.acquire() for _ in range(T)]
    st.push_ctrl(0, [L], [cur], [tmp])
    st.capture()
    for o in tmp:
        slots.release(o)
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L_start = L
    e0.record()
    for t in range(warmup, n_steps):
        step(t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    acc_mean = float(np.mean(accepted[warmup:n_steps]))
    mean_len = (L_start + L) / 2.0 + T
    step_bytes = N_ATTN * mean_len * KV_BYTES_PER_TOKEN + N_GDN * (1 + T) * GDN_BYTES_PER_LAYER // 2
    us = stack_kernel_us(st, kernel_reps)
    res = dict(workload="speculative verify: 1 sequence at %d-token context, %d drafts per step, GQA group %d "
                        "(%d query rows per KV head, MFMA path), GDN checkpoint per draft, accepted ~ U{0..%d}, "
                        "rollback by index" % (L0, T, G, G * T, T),
               steps=steps, warmup=warmup, ms_per_step=round(ms, 5), steps_per_s=round(1e3 / ms, 3),
               accepted_per_step=round(acc_mean, 4), accepted_tokens_per_s=round(acc_mean * 1e3 / ms, 2),
               algorithmic_bytes_per_step=int(step_bytes),
               hbm_gbps=round(step_bytes / (ms * 1e-3) / 1e9, 1),
               attn_partial_gbps=round(L * KV_BYTES_PER_TOKEN / (us["attn_partial"] * 1e-6) / 1e9, 1),
               us_per_layer=us, num_splits=st.n_splits)
    log("speculative: %.1f steps/s, %.2f accepted/step, partial %.1f us" % (1e3 / ms, acc_mean, us["attn_partial"]))
    check_sentinel(st)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_agentic(first_turn=50000, turns=12, turn_len=800, kernel_reps=4, seed=6):
    """Agentic multi-turn: 50,000-token first turn, then `turns` turns of
    `turn_len` decode steps.  At each turn boundary the conversation so far
    goes into the hybrid prefix cache (its pages and the current GDN state
    slot as the checkpoint) and the next turn resumes from the cache's match
    of the whole history; the next step reads the checkpoint slot and writes
    a fresh one."""
    import torch

    import hybrid_attention_decode_amd as had
    import synth

    n_steps = turns * turn_len
    max_len = first_turn + n_steps + 1
    max_pages = -(-max_len // P) + 1
    num_pages = max_pages + turns + 8        # + the partial pages the cache keeps at turn boundaries
    n_slots = turns + 4
    st = Stack(1, 1, H_Q, num_pages, max_pages, max_len, n_slots, n_steps, seed)
    pt = had.PageTable(num_pages, P, 1, max_pages, free_order=synth.permutation(num_pages, synth.seed_of(seed, 1)))
    slots = had.SlotPool(n_slots, free_order=synth.permutation(n_slots, synth.seed_of(seed, 2)))
    seq = pt.seq_create()
    pt.reserve(seq, first_turn)
    table, _ = pt.export([seq], max_pages)
    st.pt_dev.copy_(torch.from_numpy(table))
    cur = slots.acquire()
    L = first_turn
    checkpoints = []
    cache = had.RadixCache(pt, slots)
    tokens = np.zeros(max_len + 1, dtype=np.int32)                   # synthetic token ids of the conversation
    tokens[:first_turn] = synth.integers(0, 150000, first_turn, synth.seed_of(seed, 3))
    tok_rng = np.random.default_rng(synth.seed_of(seed, 4))
    locks = []
    host_us = []
    n_cow = [0]

    def step(t):
        nonlocal cur, L
        if t > 0 and t % turn_len == 0:            # turn boundary: cache the conversation, resume from the cache
            h0 = time.perf_counter()
            row = pt.export([seq], max_pages)[0][0]
            cache.insert(tokens[:L], row[:-(-L // P)], cur)
            tokens[L] = tok_rng.integers(0, 150000)    # the next turn: the whole history plus its first new token
            m, slot, pages, lock = cache.match(tokens[:L + 1])
            if m != L or slot != cur or list(pages) != list(row[:-(-L // P)]):
                raise RuntimeError("prefix cache did not return the cached conversation")
            locks.append(lock)
            host_us.append((time.perf_counter() - h0) * 1e6)
            checkpoints.append(cur)
        tokens[L] = tok_rng.integers(0, 150000)
        out = slots.acquire()
        trip = pt.reserve(seq, 1)
        L += 1
        if trip is not None:                       # the cache shares the partial last page: the step copies it
            n_cow[0] += 1
        if trip is not None or (L - 1) % P == 0:
            st.set_page(0, (L - 1) // P, pt.export([seq], max_pages)[0][0, (L - 1) // P])
        st.push_ctrl(t, [L], [cur], [[out]], cow=[trip])
        st.replay(trip is not None)
        slots.release(cur)
        cur = out

    st.push_ctrl(0, [L], [cur], [[cur]])   # capture's eager run: mapped pages only, in-place T = 1
    st.capture()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(turns + 1)]
    e0.record()
    for t in range(n_steps):
        if t % turn_len == 0:
            ev[t // turn_len].record()
        step(t)
    ev[turns].record()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    per_turn = [ev[i].elapsed_time(ev[i + 1]) / turn_len for i in range(turns)]
    mean_len = first_turn + (n_steps + 1) / 2.0
    step_bytes = algorithmic_bytes_per_step(mean_len)
    us = stack_kernel_us(st, kernel_reps)
    res = dict(workload="agentic multi-turn: %d-token first turn, %d turns x %d decode steps (context %d -> %d); at "
                        "every turn boundary the conversation goes into the hybrid prefix cache (pages + GDN "
                        "checkpoint slot) and the next turn resumes from its match" % (
                            first_turn, turns, turn_len, first_turn + 1, first_turn + n_steps),
               steps=n_steps, ms_per_step=round(ms, 5), steps_per_s=round(1e3 / ms, 3),
               first_turn_steps_per_s=round(1e3 / per_turn[0], 2), last_turn_steps_per_s=round(1e3 / per_turn[-1], 2),
               checkpoints_kept=len(checkpoints), algorithmic_bytes_per_step=int(step_bytes),
               hbm_gbps=round(step_bytes / (ms * 1e-3) / 1e9, 1), us_per_layer_at_end=us)
    cst = cache.stats()
    res["prefix_cache"] = dict(turn_boundaries=len(host_us), hit_rate=round(cst["matched_tokens"] / cst["queried_tokens"], 5),
                               nodes=cst["nodes"], checkpoints=cst["checkpoints"], cached_tokens=cst["cached_tokens"],
                               host_us_per_boundary=round(float(np.mean(host_us)), 1),
                               host_us_per_boundary_median=round(float(np.median(host_us)), 1),
                               host_us_per_boundary_max=round(float(np.max(host_us)), 1), cow_copies=n_cow[0])
    for lk in locks:
        cache.unlock(lk)
    cache.close()
    log("agentic: %.1f steps/s over %d steps; prefix cache hit rate %.4f, host work per turn boundary %.0f us "
        "(median %.0f, max %.0f)" % (1e3 / ms, n_steps, res["prefix_cache"]["hit_rate"],
                                     res["prefix_cache"]["host_us_per_boundary"],
                                     res["prefix_cache"]["host_us_per_boundary_median"],
                                     res["prefix_cache"]["host_us_per_boundary_max"]))
    check_sentinel(st)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_prefix_shared(n_seqs=16, prefix=50000, max_suffix=12288, steps=256, warmup=10, kernel_reps=4, seed=7,
                      cascade=True):
    """Prefix-shared concurrency: n_seqs sequences fork one prefix (page
    aliasing, copy-on-write of the shared partial page on first append), private
    suffixes ~ U{0..max_suffix}, GDN input slots drawn as a permutation
    (sequences without a suffix read the shared prefix checkpoint).  With
    cascade, attention reads the prefix's whole pages once for all sequences."""
    import torch

    import hybrid_attention_decode_amd as had
    import synth

    n_steps = steps + warmup
    suffix = synth.integers(0, max_suffix, n_seqs, synth.seed_of(seed, 4))
    max_len = prefix + int(suffix.max()) + n_steps + 2
    max_pages = -(-max_len // P) + 1
    prefix_pages = -(-prefix // P)
    num_pages = prefix_pages + sum(-(-(int(x) + n_steps + P) // P) + 1 for x in suffix) + 16
    n_slots = 64
    st = Stack(n_seqs, 1, H_Q, num_pages, max_pages, max_len, n_slots, n_steps, seed)
    pt = had.PageTable(num_pages, P, n_seqs + 1, max_pages,
                       free_order=synth.permutation(num_pages, synth.seed_of(seed, 1)))
    root = pt.seq_create()
    pt.reserve(root, prefix)                                  # the cached prefix
    seqs = [pt.seq_fork(root, prefix) for _ in range(n_seqs)]
    n_cow = 0

    def cow(trip):                                            # set-up time copies (eager)
        nonlocal n_cow
        if trip is None:
            return False
        for a in st.attn:
            had.kv_copy_pages(a["k_pool"], a["v_pool"], [trip[0]], [trip[1]], d_err=st.err)
        n_cow += 1
        return True

    for i, sq in enumerate(seqs):                             # private suffixes (raw append)
        if suffix[i] > 0:
            cow(pt.reserve(sq, int(suffix[i])))
    table, lens = pt.export(seqs, max_pages)
    st.pt_dev.copy_(torch.from_numpy(table))
    if cascade:                                               # the prefix's whole pages, shared by every fork
        st.enable_cascade(torch.from_numpy(table[0, :prefix // P].copy()).to("cuda"))
    slot_order = synth.permutation(n_slots, synth.seed_of(seed, 2))
    slots = had.SlotPool(n_slots, free_order=slot_order)
    shared = slots.acquire()                                  # prefix checkpoint
    cur = []
    for i in range(n_seqs):
        if suffix[i] == 0:
            slots.retain(shared)
            cur.append(shared)
        else:
            cur.append(slots.acquire())
    Ls = [int(x) for x in lens]

    def step(t):
        nonlocal n_cow
        outs = [slots.acquire() for _ in range(n_seqs)]
        trips = []
        for i, sq in enumerate(seqs):
            pos = Ls[i]
            trip = pt.reserve(sq, 1)                    # a shared partial page is copied inside the step
            trips.append(trip)
            Ls[i] += 1
            if trip is not None or pos % P == 0:        # the token's page entry changed
                st.set_page(i, pos // P, pt.export([sq], max_pages)[0][0, pos // P])
        n_step_cow = sum(x is not None for x in trips)
        n_cow += n_step_cow
        st.push_ctrl(t, Ls, cur, [[o] for o in outs], cow=trips)
        st.replay(n_step_cow > 0)
        for i in range(n_seqs):
            slots.release(cur[i])
            cur[i] = outs[i]

    tmp = [slots.acquire() for _ in range(n_seqs)]            # distinct slots for the capture run
    # its eager run reads mapped pages only (it rewrites each sequence's last held row
    # with the synthetic new-token K/V; the values do not affect timing)
    st.push_ctrl(0, Ls, cur, [[o] for o in tmp])
    st.capture()
    for o in tmp:
        slots.release(o)
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L0s = list(Ls)
    e0.record()
    for t in range(warmup, n_steps):
        step(t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    mean_lens = [(a + b) / 2.0 for a, b in zip(L0s, Ls)]
    logical = N_ATTN * sum(mean_lens) * KV_BYTES_PER_TOKEN + N_GDN * n_seqs * GDN_BYTES_PER_LAYER
    unique = N_ATTN * (prefix + sum(m - prefix for m in mean_lens)) * KV_BYTES_PER_TOKEN + \
        N_GDN * n_seqs * GDN_BYTES_PER_LAYER
    us = stack_kernel_us(st, kernel_reps)
    res = dict(workload="prefix-shared: %d sequences fork a %d-token prefix (copy-on-write on the first divergent "
                        "page), private suffixes ~ U{0..%d}, %d GDN slots, one token per sequence per step; attention %s"
                        % (n_seqs, prefix, max_suffix, n_slots,
                           "reads the prefix's whole pages once for all sequences (cascade: prefix and suffix passes in one "
                           "launch, units split by length on the device)" if cascade
                           else "per sequence (fused prologue + split-K)"),
               steps=steps, warmup=warmup, ms_per_step=round(ms, 5), steps_per_s=round(1e3 / ms, 3),
               tokens_per_s=round(n_seqs * 1e3 / ms, 2), cow_copies=n_cow,
               logical_bytes_per_step=int(logical), unique_bytes_per_step=int(unique),
               logical_gbps=round(logical / (ms * 1e-3) / 1e9, 1), unique_gbps=round(unique / (ms * 1e-3) / 1e9, 1),
               us_per_layer=us, num_splits=st.n_splits)
    log("prefix-shared (%s): %.1f steps/s (%.0f tokens/s), %d CoW copies" % (
        "cascade" if cascade else "per sequence", 1e3 / ms, n_seqs * 1e3 / ms, n_cow))
    check_sentinel(st)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_gdn_prefill(lengths=(800, 50000), reps=10, seed=8):
    """GDN half of a prefill: one sequence's prompt through one GDN layer (8
    heads, d_k = d_v = 128, raw gates) by the chunk-parallel kernels -- the
    agentic workload's 800-token turn inputs and its 50,000-token first
    turn.  Per-kernel times come from a rocprofv3 kernel trace; here the
    whole call is timed (graph of `reps` back-to-back calls)."""
    import torch

    import hybrid_attention_decode_amd as had
    import synth

    dev = "cuda"
    res = {}
    for N in lengths:
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed_of(seed, N))
        q = torch.randn((N, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
        k = torch.randn((N, GDN_H, DK), generator=g, device=dev, dtype=torch.float64)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v = torch.randn((N, GDN_H, DV), generator=g, device=dev, dtype=torch.bfloat16)
        gg = -0.1 * torch.rand((N, GDN_H), generator=g, device=dev)
        bb = torch.randn((N, GDN_H), generator=g, device=dev)
        pool = torch.randn((2, GDN_H, DV, DK), generator=g, device=dev) * 0.05
        cu = torch.tensor([0, N], dtype=torch.int32, device=dev)
        i_in = torch.tensor([0], dtype=torch.int32, device=dev)
        i_out = torch.tensor([1], dtype=torch.int32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        desc = had.gdn_prefill_desc(pool.shape, 1, N, raw_gates=True)
        ws = torch.empty(had.gdn_prefill_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        o = torch.empty((N, GDN_H, DV), device=dev)

        def call(r):
            had.gdn_prefill(pool, i_in, i_out, cu, q, k, v, gg, bb, max_len=N, o=o, workspace=ws, d_err=err,
                            raw_gates=True)

        us = time_graph(torch, call, reps)
        if int(err.item()):
            raise RuntimeError("gdn_prefill reported error bits 0x%x" % int(err.item()))
        chunks = -(-N // 64)
        res[str(N)] = dict(tokens=N, us_per_layer=round(us, 2), tokens_per_s_per_layer=round(N / (us * 1e-6), 0),
                           us_per_chunk=round(us / chunks, 3), workspace_mb=round(ws.numel() / 1e6, 1),
                           gdn_layers_of_the_stack_ms=round(N_GDN * us * 1e-3, 3))
        log("gdn prefill %d tokens: %.1f us per layer (%.3f us per 64-token chunk)" % (N, us, us / chunks))
        del q, k, v, gg, bb, pool, ws, o
        torch.cuda.empty_cache()
    return dict(workload="GDN prefill of one prompt through one layer (8 heads, d_k = d_v = 128, raw gates): "
                         "the 800-token turn input and the 50,000-token first turn of the agentic loop", **res)


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling the PMC byte counters."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: %d bytes read, %d bytes written" % (nbytes, nbytes))


def roofline(res):
    r = dict(bound="hbm", achieved=round(res["attn_partial_gbps"], 1), peak=PEAK_HBM_GBPS, unit="GB/s",
             frac=round(res["attn_partial_gbps"] / PEAK_HBM_GBPS, 4), traffic=None,
             kernel="attn_valu_kernel<256, true> (prologue fused)", bytes_per_launch=res["attn_partial_bytes_per_launch"],
             context=res["attn_partial_context"])
    try:
        with open(PMC_SUMMARY) as f:
            pmc = json.load(f)
        if pmc.get("kernel_sources_sha256") == kernel_source_hash() and pmc.get("context") == res["context"]:
            r["traffic"] = pmc.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return r


def cpu_cores():
    """Host threads: the OS count, the ones this process may run on, and the
    BLAS pool the oracle's matrix products use (its other steps run on one)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = 1
    return dict(os=os.cpu_count(), affinity=len(os.sched_getaffinity(0)), blas_threads=int(blas))


def cpu_baseline(workload, min_seconds=6.0, max_blocks=1000, seed=0):
    """The fp64 oracle timed on the host on one block of the workload's stack
    (1 attention layer with its prologue + 3 GDN layers, the 3:1 ratio), repeated
    for >= min_seconds and scaled x12 to the 48-layer step.  The attention
    layer's prior context is random bf16 drawn on the device (the benchmark's
    distribution) and copied to the host once; the oracle's gather through a
    shuffled page table is part of what is timed.

    workload: ("longctx", L0) -- 1 sequence at context L0, 8 query rows;
    ("speculative", L0) -- 1 sequence, 4 drafts x 16 query heads, GDN 4
    checkpoints; ("agentic", L) -- 1 sequence at context L; ("prefix", n,
    prefix, suffixes) -- n sequences sharing a prefix's pages."""
    import torch

    import synth
    from oracle import attention as A
    from oracle import bf16, gdn
    from oracle import prologue as Pr

    kind = workload[0]
    rng = np.random.default_rng(seed)
    T, H_q, n_seqs = 1, H_Q, 1
    if kind in ("longctx", "agentic"):
        lens = [workload[1] + 1]
    elif kind == "speculative":
        T, H_q = 4, 16
        lens = [workload[1] + T]
    else:
        n_seqs, prefix, suffixes = workload[1], workload[2], workload[3]
        lens = [prefix + int(x) + 1 for x in suffixes]
    # pages: a shared prefix (prefix-shared workload) then private pages, shuffled
    shared = workload[2] // P if kind == "prefix" else 0
    own = [-(-L // P) - shared for L in lens]
    n_pages = shared + sum(own)
    perm = rng.permutation(n_pages).astype(np.int32)
    max_pages = max(-(-L // P) for L in lens)
    table = np.full((n_seqs, max_pages), -1, np.int32)
    at = shared
    for i in range(n_seqs):
        table[i, :shared] = perm[:shared]
        table[i, shared:shared + own[i]] = perm[at:at + own[i]]
        at += own[i]
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed_of(seed, 900))
    kb = synth.bits(torch.randn((n_pages, H_KV, P, D), generator=g, device="cuda", dtype=torch.bfloat16))
    vb = synth.bits(torch.randn((n_pages, H_KV, P, D), generator=g, device="cuda", dtype=torch.bfloat16))
    lens = np.asarray(lens, np.int32)
    qg = rng.standard_normal((n_seqs, T, H_q, 2, D))
    kn, vn = rng.standard_normal((n_seqs, T, H_KV, D)), rng.standard_normal((n_seqs, T, H_KV, D))
    w = rng.random(D) + 0.5
    n_slots = n_seqs * (T + 1)
    pool = (rng.standard_normal((n_slots, GDN_H, DV, DK)) * 0.05).astype(np.float32)
    gq = rng.standard_normal((n_seqs, T, GDN_H, DK))
    gk = rng.standard_normal((n_seqs, T, GDN_H, DK))
    gk /= np.linalg.norm(gk, axis=-1, keepdims=True)
    gv = rng.standard_normal((n_seqs, T, GDN_H, DV))
    ga, gb = rng.uniform(0.9, 1, (n_seqs, T, GDN_H)), rng.uniform(0, 1, (n_seqs, T, GDN_H))
    in_idx = np.arange(n_seqs)
    out_idx = n_seqs + np.arange(n_seqs * T).reshape(n_seqs, T)
    qb = bf16.from_f64(rng.standard_normal((n_seqs, T, H_q, D)))
    blocks = 0
    t0 = time.perf_counter()
    while blocks < max_blocks:
        for i in range(n_seqs):
            Pr.qk_norm_rope_gate(qg[i], kn[i], vn[i], w, w, np.arange(lens[i] - T, lens[i]), R)
        A.paged_attention(qb, kb, vb, table, lens, P, 1 / 16.0)
        for _ in range(3):
            gdn.state_update(pool, in_idx, out_idx, gq, gk, gv, ga, gb)
        blocks += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    per_step = el / blocks * (N_ATTN + N_GDN) / 4
    cores = cpu_cores()
    what = {"longctx": "1 sequence at context %d" % lens[0],
            "agentic": "1 sequence at context %d" % lens[0],
            "speculative": "1 sequence at context %d, %d drafts x %d query heads, GDN %d checkpoints" % (
                lens[0], T, H_q, T),
            "prefix": "%d sequences sharing a %d-token prefix, contexts %d..%d" % (
                n_seqs, shared * P, lens.min(), lens.max())}[kind]
    return dict(value=round(1.0 / per_step, 6), unit="steps/s", cores=cores["blas_threads"], kind="oracle",
                cores_os=cores["os"], cores_affinity=cores["affinity"], blas_threads=cores["blas_threads"],
                sample="%d block(s) of 1 attention layer with its prologue (%s) + 3 GDN layers in %.1f s, "
                       "scaled x12 to the 48-layer step" % (blocks, what, el))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ctx", type=int, default=131072, help="context of the headline value")
    ap.add_argument("--sweep", default="262144,1048576", help="further contexts measured in the same run")
    ap.add_argument("--kernel-reps", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="oracle timing per workload (seconds)")
    ap.add_argument("--seed", type=int, default=0, help="base seed of the synthetic inputs")
    ap.add_argument("--workloads", default="speculative,agentic,prefix,prefill",
                    help="further workloads reported beside the headline (comma list, '' for none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (scales PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: one GPU only; --gpus %d is not supported "
              "(the multi-GPU split of this path is a design note, not a code path)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import hybrid_attention_decode_amd as had

    had.lib()
    if args.copy_calibration:
        copy_calibration()
    head = run_context(args.ctx, args.steps, args.warmup, args.kernel_reps, seed=args.seed)
    sweep = []
    for c in [int(x) for x in args.sweep.split(",") if x.strip()]:
        sweep.append(run_context(c, args.steps, args.warmup, args.kernel_reps, seed=args.seed))
    extra = {}
    wl = [w.strip() for w in args.workloads.split(",") if w.strip()]
    if "speculative" in wl:
        extra["speculative"] = run_speculative(steps=args.steps, warmup=args.warmup, kernel_reps=args.kernel_reps,
                                               seed=5 + args.seed)
    if "agentic" in wl:
        extra["agentic"] = run_agentic(kernel_reps=args.kernel_reps, seed=6 + args.seed)
    if "prefix" in wl:
        extra["prefix_shared"] = run_prefix_shared(steps=args.steps, warmup=args.warmup,
                                                   kernel_reps=args.kernel_reps, seed=7 + args.seed)
        flat = run_prefix_shared(steps=args.steps, warmup=args.warmup, kernel_reps=args.kernel_reps, seed=7 + args.seed,
                                 cascade=False)
        extra["prefix_shared"]["per_sequence_path"] = {k: flat[k] for k in ("steps_per_s", "tokens_per_s",
                                                                            "us_per_layer")}
    cpu = None
    if "prefill" in wl:
        extra["gdn_prefill"] = run_gdn_prefill(seed=8 + args.seed)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(("longctx", args.ctx), args.cpu_seconds)
        log("oracle: %s" % cpu)
        # the other workloads' oracle step rates, each on its own sample
        if "speculative" in extra:
            extra["speculative"]["cpu_baseline"] = cpu_baseline(("speculative", 262144), args.cpu_seconds)
        if "agentic" in extra:
            extra["agentic"]["cpu_baseline"] = cpu_baseline(("agentic", 50000 + 4800), args.cpu_seconds)
        if "prefix_shared" in extra:
            import synth
            sfx = synth.integers(0, 12288, 16, synth.seed_of(7 + args.seed, 4))
            extra["prefix_shared"]["cpu_baseline"] = cpu_baseline(("prefix", 16, 50000, sfx), args.cpu_seconds)
        for k in ("speculative", "agentic", "prefix_shared"):
            if k in extra and "cpu_baseline" in extra[k]:
                log("oracle (%s): %s" % (k, extra[k]["cpu_baseline"]))
    out = {
        "metric": METRIC,
        "value": round(head["steps_per_s"], 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long-context decode: 1 sequence, %d-token context, %d decode steps timed, 48-layer hybrid "
                        "stack (12 full-attention: 8 q / 1 KV heads, head_dim 256, partial RoPE 64, bf16 KV in "
                        "64-token permuted pages; 36 Gated DeltaNet: 8 heads, 128x128 fp32 state)"
                        % (args.ctx, args.steps),
            "context": args.ctx,
            "parallelism": "none (1 GPU, one GPU's head share)",
        },
        "hbm_gbps": round(head["hbm_gbps"], 1),
        "hbm_frac_of_peak": round(head["hbm_frac"], 4),
        "us_per_layer": head["us_per_layer"],
        "graph_only_ms_per_step": round(head["graph_only_ms_per_step"], 5),
        "num_splits": head["num_splits"],
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in sweep],
        "workloads": extra,
        "roofline": roofline(head),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
