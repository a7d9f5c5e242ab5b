"""Pins for the oracle's page-table / slot model and the paged gather (CPU)."""

import numpy as np
import pytest

from oracle import paging
from oracle.paging import ModelError, PageTableModel, SlotPoolModel
import scenario


def test_hand_worked_scenario():
    cfg, order, ops = scenario.load("page_table_scenario.txt")
    pt = PageTableModel(*cfg, free_order=order)
    scenario.run(pt, ops, ModelError)


def _check_invariants(pt):
    refs = np.array(pt.ref)
    counted = np.zeros_like(refs)
    for s in pt.seqs.values():
        for p in s["pages"]:
            counted[p] += 1
        assert len(s["pages"]) == -(-s["len"] // pt.P)
    assert np.array_equal(refs, counted)                    # refcount conservation
    free = set(pt.free)
    assert len(free) == len(pt.free)                        # no duplicates
    assert all(refs[p] == 0 for p in free)                  # free pages are unreferenced
    assert free | {p for p in range(pt.num_pages) if refs[p] > 0} == set(range(pt.num_pages))


def test_fuzz_invariants():
    rng = np.random.default_rng(7)
    for trial in range(20):
        P = int(rng.integers(1, 9))
        N = int(rng.integers(4, 40))
        pt = PageTableModel(N, P, 6, 12, free_order=list(rng.permutation(N)))
        for _ in range(300):
            op = rng.integers(0, 6)
            sids = list(pt.seqs)
            try:
                if op == 0 or not sids:
                    pt.seq_create()
                elif op == 1:
                    src = sids[rng.integers(len(sids))]
                    n = int(rng.integers(0, pt.seqs[src]["len"] + 1))
                    before = list(pt.seqs[src]["pages"])
                    sid = pt.seq_fork(src, n)
                    assert pt.seqs[sid]["pages"] == before[: -(-n // P)]
                elif op == 2 or op == 5:
                    sid = sids[rng.integers(len(sids))]
                    snap = (list(pt.free), list(pt.ref), {k: (list(v["pages"]), v["len"]) for k, v in pt.seqs.items()})
                    L = pt.seqs[sid]["len"]
                    pages = list(pt.seqs[sid]["pages"])
                    try:
                        r = pt.reserve(sid, int(rng.integers(0, 2 * P + 1)))
                    except ModelError:
                        # transactional: nothing changed
                        assert snap == (pt.free, pt.ref, {k: (v["pages"], v["len"]) for k, v in pt.seqs.items()})
                        continue
                    if r is not None:
                        src, dst, valid = r
                        assert src == pages[-1] and valid == L % P and valid > 0
                        assert pt.seqs[sid]["pages"][len(pages) - 1] == dst
                elif op == 3:
                    sid = sids[rng.integers(len(sids))]
                    pt.truncate(sid, int(rng.integers(0, pt.seqs[sid]["len"] + 1)))
                else:
                    pt.seq_free(sids[rng.integers(len(sids))])
            except ModelError as e:
                assert e.kind in ("capacity", "out_of_pages")
            _check_invariants(pt)


def test_slots_policy():
    sp = SlotPoolModel(4, free_order=[2, 0, 3, 1])
    assert sp.acquire() == 1
    assert sp.acquire() == 3
    sp.retain(1)
    sp.release(1)
    assert sp.stats() == (2, 2)
    sp.release(1)
    assert sp.free == [2, 0, 1]
    with pytest.raises(ModelError) as e:
        sp.release(1)
    assert e.value.kind == "bad_slot"
    assert sp.acquire() == 1
    assert sp.acquire() == 0
    assert sp.acquire() == 2
    with pytest.raises(ModelError) as e:
        sp.acquire()
    assert e.value.kind == "out_of_slots"


def test_gather_is_inverse_of_scatter_bit_exact():
    rng = np.random.default_rng(3)
    P, H, D, L = 16, 2, 8, 77
    n_pages = -(-L // P)
    rows = rng.integers(0, 65536, size=(L, H, D), dtype=np.uint16)
    for pages in (np.arange(n_pages), rng.permutation(40)[:n_pages]):
        pool = rng.integers(0, 65536, size=(40, H, P, D), dtype=np.uint16)
        paging.scatter_contiguous(rows, pages, P, pool)
        assert np.array_equal(paging.gather(pool, pages, L, P), rows)
        assert np.array_equal(paging.gather(pool, pages, L, P, head=1), rows[:, 1])


def test_gather_reads_the_addressed_page_slot():
    # position t lives at pool[pages[t // P], h, t % P]: check one element by hand
    pool = np.arange(5 * 1 * 4 * 2).reshape(5, 1, 4, 2)
    pages = [3, 0, 4]
    g = paging.gather(pool, pages, 10, 4)
    assert g[5, 0, 1] == pool[0, 0, 1, 1]
    assert g[9, 0, 0] == pool[4, 0, 1, 0]
    assert g[2, 0, 1] == pool[3, 0, 2, 1]
