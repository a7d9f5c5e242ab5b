"""Pins for the oracle's draft rollback model (CPU)."""

import numpy as np
import pytest

from oracle import attention as A
from oracle import gdn, paging, speculative
from oracle.paging import ModelError, PageTableModel, SlotPoolModel


def _setup(L0, T):
    pt = PageTableModel(32, 4, 4, 16, free_order=list(np.random.default_rng(0).permutation(32)))
    sp = SlotPoolModel(8, free_order=[3, 7, 0, 5, 1, 6, 2, 4])
    sid = pt.seq_create()
    pt.reserve(sid, L0)
    cur = sp.acquire()
    pt.reserve(sid, T)
    outs = [sp.acquire() for _ in range(T)]
    return pt, sp, sid, cur, outs


@pytest.mark.parametrize("a", [0, 1, 2, 3, 4])
def test_rollback_bookkeeping(a):
    L0, T = 10, 4
    pt, sp, sid, cur, outs = _setup(L0, T)
    keep = speculative.rollback(pt, sp, sid, T, a, cur, outs)
    assert keep == (cur if a == 0 else outs[a - 1])
    assert pt.seqs[sid]["len"] == L0 + a
    held = {s for s in range(8) if sp.ref[s] > 0}
    assert held == {keep}
    # pages beyond the kept length went back to the free list
    assert len(pt.seqs[sid]["pages"]) == -(-(L0 + a) // 4)


def test_rollback_is_transactional():
    pt, sp, sid, cur, outs = _setup(10, 4)
    snap = (list(pt.free), list(pt.ref), list(sp.free), list(sp.ref))
    for bad in ([outs[0]] * 4, outs[:3] + [cur]):
        with pytest.raises(ModelError):
            speculative.rollback(pt, sp, sid, 4, 2, cur, bad)
        assert snap == (pt.free, pt.ref, sp.free, sp.ref)
    with pytest.raises(ModelError):
        speculative.rollback(pt, sp, sid, 4, 5, cur, outs)
    assert snap == (pt.free, pt.ref, sp.free, sp.ref)


def test_after_rollback_results_equal_the_never_drafted_run():
    rng = np.random.default_rng(1)
    L0, T, a, D, Hq = 13, 4, 2, 8, 4
    ctx_k = rng.standard_normal((L0, 1, D))
    ctx_v = rng.standard_normal((L0, 1, D))
    drafts_k = rng.standard_normal((T, 1, D))
    drafts_v = rng.standard_normal((T, 1, D))
    nxt_k, nxt_v = rng.standard_normal((1, 1, D)), rng.standard_normal((1, 1, D))
    q = rng.standard_normal((1, Hq, D))
    # drafted: T tokens written at L0..L0+3, then truncated to L0+a, next token
    # overwrites position L0+a (stale K/V beyond the length is never read)
    k_buf = np.concatenate([ctx_k, drafts_k])
    v_buf = np.concatenate([ctx_v, drafts_v])
    k_buf[L0 + a] = nxt_k[0]
    v_buf[L0 + a] = nxt_v[0]
    o_drafted = A.attention(q, k_buf[: L0 + a + 1], v_buf[: L0 + a + 1], 0.3)
    k_ref = np.concatenate([ctx_k, drafts_k[:a], nxt_k])
    v_ref = np.concatenate([ctx_v, drafts_v[:a], nxt_v])
    assert np.array_equal(o_drafted, A.attention(q, k_ref, v_ref, 0.3))
    # GDN: the state after accepting a drafts is the checkpoint of draft a-1
    S0 = rng.standard_normal((D, D))
    gq, gk = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    gk /= np.linalg.norm(gk, axis=1, keepdims=True)
    gv = rng.standard_normal((T, D))
    al, be = rng.uniform(0.9, 1, T), rng.uniform(0, 1, T)
    st, _ = gdn.sequential(S0, gq, gk, gv, al, be)
    st_a, _ = gdn.sequential(S0, gq[:a], gk[:a], gv[:a], al[:a], be[:a])
    assert np.array_equal(st[a - 1], st_a[-1])
