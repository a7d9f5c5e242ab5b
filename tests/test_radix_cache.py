"""Hybrid prefix cache (C++ radix tree with state-slot checkpoints) against
the brute-force model, on the CPU.

Every physical page's rows and every state slot's "state" (the token
sequence it summarises) are simulated on the host, so a lookup is checked
by content: the pages it returns must hold the matched tokens, and its slot
must hold the state of exactly the matched prefix.
"""

import ctypes

import numpy as np
import pytest

import hybrid_attention_decode_amd as had
from oracle.radix import PrefixCacheModel


def test_model_hand_cases():
    m = PrefixCacheModel()
    m.insert([1, 2, 3], 7)
    m.insert([1, 2, 3, 4, 5], 9)
    m.insert([1, 2, 3], 8)       # saved again: the first state stays
    m.insert([4, 4], -1)         # no state: not a resume point
    assert m.match([1, 2, 3, 4, 9]) == (3, 7)
    assert m.match([1, 2, 3, 4, 5, 6]) == (5, 9)
    assert m.match([1, 2, 3, 4, 5]) == (5, 9)
    assert m.match([1, 2]) == (0, -1)
    assert m.match([4, 4, 4]) == (0, -1)
    assert m.match([]) == (0, -1)


class Sim:
    """Requests on the C++ page table, slot pool and prefix cache, with the
    content of every page row and slot simulated on the host."""

    def __init__(self, num_pages=512, P=4, n_slots=64, max_seqs=8, max_pages=200, seed=0):
        rng = np.random.default_rng(seed)
        self.P = P
        self.pt = had.PageTable(num_pages, P, max_seqs, max_pages, free_order=rng.permutation(num_pages))
        self.slots = had.SlotPool(n_slots, free_order=rng.permutation(n_slots))
        self.cache = had.RadixCache(self.pt, self.slots)
        self.model = PrefixCacheModel()
        self.rows = {}    # page -> list of P tokens (None = never written)
        self.state = {}   # slot -> tuple of the tokens it summarises
        self.max_pages = max_pages

    def _write(self, seq, pos, tok):
        page = self.pt.export([seq], self.max_pages)[0][0][pos // self.P]
        self.rows.setdefault(int(page), [None] * self.P)[pos % self.P] = int(tok)

    def _append(self, seq, toks, start):
        cow = self.pt.reserve(seq, len(toks))
        if cow is not None:              # the device half of copy-on-write: copy the valid rows
            src, dst, valid = cow
            self.rows[dst] = list(self.rows[src][:valid]) + [None] * (self.P - valid)
        for j, t in enumerate(toks):
            self._write(seq, start + j, t)

    def check_match(self, tokens, m, slot, pages):
        assert len(pages) == -(-m // self.P)
        for pos in range(m):
            assert self.rows[pages[pos // self.P]][pos % self.P] == tokens[pos], (pos, m)
        if m > 0:
            assert self.state[slot] == tuple(tokens[:m])
        else:
            assert slot == -1

    def request(self, tokens, n_generate, rng, save=True, keep_lock=False):
        """Resume from the cache, prefill the rest, decode n_generate tokens,
        save the whole sequence with its final state."""
        m, slot, pages, lock = self.cache.match(tokens)
        self.check_match(tokens, m, slot, pages)
        seq = self.pt.seq_create_from(pages, m) if m > 0 else self.pt.seq_create()
        self._append(seq, tokens[m:], m)
        full = list(tokens)
        for _ in range(n_generate):
            t = int(rng.integers(0, 50))
            self._append(seq, [t], len(full))
            full.append(t)
        new_slot = self.slots.acquire()
        self.state[new_slot] = tuple(full)
        if save:
            table, lens = self.pt.export([seq], self.max_pages)
            self.cache.insert(full, table[0][:-(-len(full) // self.P)], new_slot)
            self.model.insert(full, new_slot)
        self.slots.release(new_slot)     # the cache keeps its own reference
        self.pt.seq_free(seq)
        if not keep_lock:
            self.cache.unlock(lock)
        return full, m, slot, lock


def test_split_and_checkpoint_rules():
    s = Sim(P=4)
    rng = np.random.default_rng(1)
    a, _, _, _ = s.request([1, 2, 3, 4, 5, 6, 7], 0, rng)
    b, _, _, _ = s.request([1, 2, 3, 9, 9], 0, rng)          # leaves "a" inside its edge: split at depth 3
    st = s.cache.stats()
    assert st["nodes"] == 3 and st["checkpoints"] == 2 and st["cached_tokens"] == 7 + 2
    m, slot, pages, lock = s.cache.match([1, 2, 3, 8])
    assert (m, slot) == (0, -1)                              # no state saved at depth 3
    s.check_match([1, 2, 3, 8], m, slot, pages)
    c, _, _, _ = s.request([1, 2, 3], 0, rng)               # saves a state exactly at the split
    m, slot, pages, lock = s.cache.match([1, 2, 3, 8])
    assert m == 3 and slot == s.model.match([1, 2, 3, 8])[1]
    s.check_match([1, 2, 3, 8], m, slot, pages)
    s.cache.unlock(lock)
    for q in (a, b, c, a + [5], b[:4]):
        m, slot, pages, lock = s.cache.match(q)
        assert (m, slot) == s.model.match(q)
        s.check_match(q, m, slot, pages)
        s.cache.unlock(lock)


@pytest.mark.parametrize("P", [1, 4, 16])
def test_agentic_turns_match_the_model(P):
    # multi-turn conversations: every turn resends the whole history plus new
    # tokens; several conversations share system prompts
    rng = np.random.default_rng(10 + P)
    s = Sim(num_pages=4096, P=P, n_slots=256, max_pages=400, seed=P)
    systems = [list(rng.integers(0, 50, int(rng.integers(5, 30)))) for _ in range(3)]
    convs = [list(systems[i % 3]) for i in range(6)]
    matched = queried = 0
    for turn in range(40):
        i = int(rng.integers(0, len(convs)))
        q = convs[i] + list(rng.integers(0, 50, int(rng.integers(1, 12))))
        want = s.model.match(q)
        full, m, slot, lock = s.request(q, int(rng.integers(0, 10)), rng)
        assert (m, slot) == want
        matched += m
        queried += len(q)
        convs[i] = full
    st = s.cache.stats()
    assert st["matched_tokens"] == matched and st["queried_tokens"] == queried
    assert matched / queried > 0.5                     # the history is reused
    # releasing everything returns every page and slot
    s.cache.evict(4096, 256)
    assert s.cache.stats()["nodes"] == 0
    assert s.pt.stats() == (4096, 0)
    assert s.slots.stats() == (256, 0)


def test_eviction_keeps_locked_paths_and_agrees_with_the_model():
    rng = np.random.default_rng(5)
    s = Sim(num_pages=300, P=4, n_slots=40, max_pages=100, seed=5)
    held = []
    for turn in range(60):
        base = [int(rng.integers(0, 4))] * 3
        q = base + list(rng.integers(0, 50, int(rng.integers(1, 20))))
        if s.pt.stats()[0] < 60 or s.slots.stats()[0] < 4:
            s.cache.evict(120, 8)
        m_model, _ = s.model.match(q)
        full, m, slot, lock = s.request(q, int(rng.integers(0, 6)), rng, keep_lock=(turn % 7 == 0))
        assert m <= m_model                             # eviction only ever shortens a match
        if m > 0:
            assert s.model.saved.get(tuple(q[:m])) == slot
        if turn % 7 == 0 and m > 0:
            held.append((q, m, slot, lock))
    s.cache.evict(10 ** 6, 10 ** 6)                     # evict everything that is not locked
    for q, m, slot, lock in held:                       # locked paths survive, bit for bit
        m2, slot2, pages2, lock2 = s.cache.match(q)
        assert (m2, slot2) == (m, slot)
        s.check_match(q, m2, slot2, pages2)
        s.cache.unlock(lock2)
        s.cache.unlock(lock)
    s.cache.evict(10 ** 6, 10 ** 6)
    assert s.cache.stats()["nodes"] == 0
    assert s.pt.stats()[1] == 0 and s.slots.stats()[1] == 0


def test_errors_change_nothing():
    s = Sim(P=4)
    rng = np.random.default_rng(2)
    full, _, _, _ = s.request([3, 1, 4, 1, 5, 9, 2, 6], 0, rng)
    before = (s.cache.stats(), s.pt.stats(), s.slots.stats())
    never_written = [p for p in range(512) if p not in s.rows][:2]   # pages nobody holds
    with pytest.raises(had.HadError):
        s.cache.insert([7, 7, 7, 7, 7], never_written, 3)
    with pytest.raises(had.HadError):
        s.cache.unlock(12345)
    # the page buffer of a lookup is checked before anything changes
    L = had.lib()
    toks = np.array(full, dtype=np.int32)
    m, sl, lk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    pages = np.zeros(1, dtype=np.int32)
    st = L.had_radix_match(s.cache._h, toks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(toks),
                           ctypes.byref(m), ctypes.byref(sl), pages.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1,
                           ctypes.byref(lk))
    assert st == -9                                   # HAD_ERR_CAPACITY: 2 pages needed
    assert (s.cache.stats(), s.pt.stats(), s.slots.stats()) == before
