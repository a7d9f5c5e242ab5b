"""C ABI library: symbols, and the C++ page-table / slot manager against the
oracle's integer model, bit for bit (CPU only: no GPU compute is called)."""

import os
import re

import numpy as np
import pytest

import hybrid_attention_decode_amd as had
from hybrid_attention_decode_amd import HadError, PageTable, SlotPool
from oracle import speculative
from oracle.paging import ModelError, PageTableModel, SlotPoolModel
import scenario

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "had.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(had_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = had.lib()
    declared = _declared()
    assert len(declared) >= 25
    for name in declared:
        assert hasattr(L, name), name
    assert declared == had.exported_symbols()
    assert had.abi_version() == 5


def test_scenario_on_the_cpp_manager():
    cfg, order, ops = scenario.load("page_table_scenario.txt")
    pt = PageTable(*cfg, free_order=order)
    scenario.run(pt, ops, HadError)


def _call(obj, name, *args):
    try:
        return ("ok", getattr(obj, name)(*args))
    except (HadError, ModelError) as e:
        return ("err", e.kind)


def test_fuzz_cpp_manager_matches_model_bit_exact():
    rng = np.random.default_rng(11)
    for trial in range(12):
        P = int(rng.choice([1, 4, 16, 64]))
        N = int(rng.integers(8, 80))
        max_seqs = int(rng.integers(2, 8))
        max_pages = int(rng.integers(2, 16))
        order = rng.permutation(N)
        m = PageTableModel(N, P, max_seqs, max_pages, free_order=list(order))
        c = PageTable(N, P, max_seqs, max_pages, free_order=order)
        for step in range(400):
            op = int(rng.integers(0, 7))
            sid = int(rng.integers(-1, max_seqs + 1))
            n = int(rng.integers(0, 3 * P + 2))
            if op == 0:
                a, b = _call(m, "seq_create"), _call(c, "seq_create")
            elif op == 1:
                a, b = _call(m, "seq_fork", sid, n), _call(c, "seq_fork", sid, n)
            elif op in (2, 3):
                a, b = _call(m, "reserve", sid, n), _call(c, "reserve", sid, n)
            elif op == 4:
                L = m.seqs[sid]["len"] if sid in m.seqs else 0
                k = int(rng.integers(0, L + 2))
                a, b = _call(m, "truncate", sid, k), _call(c, "truncate", sid, k)
            elif op == 5:
                a, b = _call(m, "seq_free", sid), _call(c, "seq_free", sid)
            else:
                a, b = _call(m, "stats"), _call(c, "stats")
            assert a == b, (trial, step, op, a, b)
            live = sorted(m.seqs)
            pm, lm = m.export(live, max_pages)
            pc, lc = c.export(live, max_pages)
            assert np.array_equal(pm, pc) and np.array_equal(lm, lc)
            assert m.stats() == c.stats()


def test_fuzz_slots_and_rollback_match_model():
    rng = np.random.default_rng(12)
    for trial in range(10):
        n_slots = 16
        order = rng.permutation(n_slots)
        ms, cs = SlotPoolModel(n_slots, list(order)), SlotPool(n_slots, order)
        mp, cp = PageTableModel(64, 4, 4, 32, list(range(64))), PageTable(64, 4, 4, 32)
        sm, sc = mp.seq_create(), cp.seq_create()
        assert sm == sc
        mp.reserve(sm, 9)
        cp.reserve(sc, 9)
        for step in range(200):
            op = int(rng.integers(0, 4))
            if op == 0:
                a, b = _call(ms, "acquire"), _call(cs, "acquire")
            elif op == 1:
                x = int(rng.integers(-1, n_slots + 1))
                a, b = _call(ms, "retain", x), _call(cs, "retain", x)
            elif op == 2:
                x = int(rng.integers(-1, n_slots + 1))
                a, b = _call(ms, "release", x), _call(cs, "release", x)
            else:
                T = int(rng.integers(1, 5))
                acc = int(rng.integers(0, T + 2))
                held = [s for s in range(n_slots) if ms.ref[s] > 0]
                if len(held) < T + 1:
                    continue
                pick = list(rng.choice(held, T + 1, replace=False))
                in_slot = int(pick[0]) if rng.random() < 0.8 else -1
                outs = [int(x) for x in pick[1:]]
                if rng.random() < 0.1:
                    outs[0] = outs[-1]  # invalid: repeated
                mp.reserve(sm, T)
                cp.reserve(sc, T)
                try:
                    a = ("ok", speculative.rollback(mp, ms, sm, T, acc, in_slot, outs))
                except ModelError as e:
                    a = ("err", e.kind)
                try:
                    b = ("ok", had.spec_rollback(cp, cs, sc, T, acc, in_slot, outs))
                except HadError as e:
                    b = ("err", e.kind)
            assert a == b, (trial, step, a, b)
            assert ms.stats() == cs.stats()
            assert mp.export([sm], 32)[0].tolist() == cp.export([sc], 32)[0].tolist()
            assert mp.export([sm], 32)[1].tolist() == cp.export([sc], 32)[1].tolist()


def test_error_paths_leave_handles_unchanged():
    pt = PageTable(4, 4, 2, 2)
    s = pt.seq_create()
    pt.reserve(s, 5)
    before = (pt.export([s], 2), pt.stats())
    for bad in (lambda: pt.reserve(s, 4), lambda: pt.truncate(s, 6), lambda: pt.seq_fork(s, 9),
                lambda: pt.reserve(9, 1), lambda: pt.export([s], 1)):
        with pytest.raises(HadError):
            bad()
    after = (pt.export([s], 2), pt.stats())
    assert np.array_equal(before[0][0], after[0][0]) and before[1] == after[1]
    with pytest.raises(HadError) as e:
        PageTable(4, 4, 2, 2, free_order=[0, 1, 1, 3])
    assert e.value.kind == "invalid"
    assert "free_order" in str(e.value)


def test_gdn_slot_precondition_checker():
    ok = [([0, 1], [[2], [3]], False), ([0, -1], [[0], [3]], True), ([4, 4], [[1, 2], [3, 0]], False),
          ([-1], [[0, 1, 2, 3]], False)]
    for in_idx, out_idx, inplace in ok:
        had.gdn_check_slots(6, np.array(in_idx), np.array(out_idx), inplace)
    bad = [([0, 1], [[2], [2]], False),        # one slot written twice
           ([0, 2], [[2], [3]], False),        # written by sequence 0, read by sequence 1
           ([0], [[0]], False),                # in place where not allowed
           ([0], [[6]], True),                 # out of range
           ([-2], [[1]], True),                # in out of range
           ([1, 0], [[1, 2], [3, 4]], False)]  # a checkpoint slot that is the input: not in place
    for in_idx, out_idx, inplace in bad:
        with pytest.raises(HadError) as e:
            had.gdn_check_slots(6, np.array(in_idx), np.array(out_idx), inplace)
        assert e.value.kind == "bad_slot", (in_idx, out_idx)


def _prefill_segments(n_seqs, H, dk, dv, max_len, n_segments=0):
    """Segments the prefill plans, read back from its workspace size (host
    call, no GPU): the segmented layout adds n_seqs x G x H blocks of
    (d_k x d_k + 2 x d_v x d_k) floats after the 256-byte-aligned chunk part."""
    one = had.gdn_prefill_workspace_bytes(had.gdn_prefill_desc((1, H, dv, dk), n_seqs, max_len, n_segments=1))
    got = had.gdn_prefill_workspace_bytes(had.gdn_prefill_desc((1, H, dv, dk), n_seqs, max_len,
                                                               n_segments=n_segments))
    extra = got - one
    per = n_seqs * H * (dk * dk + 2 * dv * dk) * 4
    assert extra % per == 0
    return 1 if extra == 0 else extra // per


def test_prefill_segment_plan():
    assert _prefill_segments(1, 8, 128, 128, 50000) == 8       # 782 chunks, 64 one-pass workgroups
    assert _prefill_segments(1, 8, 128, 128, 800) == 1         # 13 chunks: one pass
    assert _prefill_segments(1, 2, 128, 128, 6144) == 3        # 96 chunks
    assert _prefill_segments(1, 2, 128, 128, 4096) == 1        # two segments would gain nothing
    assert _prefill_segments(16, 8, 128, 128, 50000) == 1      # the batch already fills the GPU
    assert _prefill_segments(1, 8, 128, 128, 800, n_segments=5) == 5
    assert _prefill_segments(1, 8, 128, 128, 800, n_segments=100) == 13   # capped at the chunk count
    with pytest.raises(HadError):
        had.gdn_prefill_workspace_bytes(had.gdn_prefill_desc((1, 8, 128, 128), 1, 800, n_segments=-1))


def test_attention_split_plan():
    # the benchmark's shapes (head_dim 256, 64-token pages, 1 KV head): one
    # split per CU from 128K on, for 8 rows (VALU) and 64 rows (MFMA);
    # short contexts keep >= 4 tiles of 8 tokens per wave (VALU) or >= 4
    # iterations of 64 tokens (MFMA) per split
    def plan(q_shape, max_len):
        pages = -(-max_len // 64) + 1
        return had.decode_attn_plan(had.attn_desc(q_shape, (pages, 1, 64, 256), pages, max_seq_len=max_len))
    assert plan((1, 1, 8, 256), 131072 + 266) == (256, 9)
    assert plan((1, 1, 8, 256), 262144 + 266) == (256, 17)
    assert plan((1, 1, 8, 256), 1048576 + 266) == (256, 65)
    assert plan((1, 4, 16, 256), 262144 + 1034) == (256, 17)
    assert plan((1, 1, 8, 256), 513) == (2, 5)
    assert plan((1, 4, 16, 256), 2000) == (8, 4)       # 32 pages, 4 per split
    assert plan((1, 4, 16, 256), 640) == (3, 4)        # 10 pages: 3 splits of <= 4, not 2 of 5
    # cascade: 16 sequences on a 781-page prefix (prefix pass: 196 splits of
    # <= 4 pages -- 195 would leave one of 5), suffixes up to 12,288 tokens:
    # 256 suffix units shared out by length, so every sequence's workspace
    # row has 196 + 256 slots
    n, rows, D = 16, 8, 256
    max_len = 50000 + 12288 + 300
    pages = -(-max_len // 64) + 1
    desc = had.attn_desc((n, 1, 8, D), (4096, 1, 64, D), pages, max_seq_len=max_len)
    assert had.decode_attn_cascade_plan(desc, 781) == (196, 256)
    ws = had.decode_attn_cascade_workspace_bytes(desc, 781)
    assert ws == n * 1 * (196 + 256) * rows * (D + 2) * 4
    # the per-sequence plan where the shares do not apply: 16 rows or more
    # (MFMA suffix pass), more than 64 sequences, or a forced split count
    d16 = had.attn_desc((n, 2, 8, D), (4096, 1, 64, D), pages, max_seq_len=max_len)
    assert had.decode_attn_cascade_plan(d16, 781)[1] == 16
    d65 = had.attn_desc((65, 1, 8, D), (8192, 1, 64, D), pages, max_seq_len=max_len)
    assert had.decode_attn_cascade_plan(d65, 781)[1] == 4


def test_split_page_cap_applies_to_tile_ranges_only():
    # below 16 rows a split's tile range can straddle one page more than its
    # share, so ceil(n / ns) <= 511 when ns > 1; the MFMA path's ranges are
    # whole pages and may hold 512
    def plan(q_shape, pages, ns):
        return had.decode_attn_plan(had.attn_desc(q_shape, (pages + 2, 1, 64, 64), pages, num_splits=ns))
    assert plan((1, 1, 4, 64), 1532, 3) == (3, 511)          # split 1 touches pages 510..1021: 512 ids
    with pytest.raises(HadError):
        plan((1, 1, 4, 64), 1024, 2)                          # 512 pages per split, a range could need 513
    assert plan((1, 4, 16, 64), 1024, 2) == (2, 512)         # MFMA: page ranges, 512 allowed
    with pytest.raises(HadError):
        plan((1, 4, 16, 64), 1026, 2)                         # 513 pages per split
    assert plan((1, 1, 4, 64), 512, 1) == (1, 512)           # one split reads the whole range


def test_page_copy_list_check():
    ok = [([3, -1, 5], [7, 0, 8]), ([], []), ([-1, -1], [3, 3])]
    for src, dst in ok:
        had.kv_check_copy_pages(10, src, dst)
    bad = [([3], [10]),            # destination out of range
           ([-2], [1]),            # only -1 marks an unused entry
           ([3, 4], [4, 5]),       # 4 is a destination and a source
           ([3, 4], [6, 6]),       # destination repeated
           ([3], [3])]             # copy onto itself
    for src, dst in bad:
        with pytest.raises(HadError):
            had.kv_check_copy_pages(10, src, dst)
    with pytest.raises(ValueError):
        had.kv_check_copy_pages(10, [1, 2], [3])


def test_cascade_prefix_check():
    pt = np.array([[4, 9, 2, 7], [4, 9, 5, -1], [4, 9, 2, 1]], np.int32)
    had.attn_check_prefix(pt, [4, 9])
    with pytest.raises(HadError, match="sequence 1"):
        had.attn_check_prefix(pt, [4, 9, 2])                 # sequence 1's third page was copied on write
    with pytest.raises(HadError):
        had.attn_check_prefix(pt, [4, 8])
    with pytest.raises(HadError):
        had.attn_check_prefix(pt, [4, 9, 2, 7, 0])           # longer than a row
