"""Integer model of the paged KV cache and the recurrent-state slot pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* zubnet.ai TokenSpeed article (Spanish, and its French twin), second
  paragraph: the prefix cache spans KV pages and Mamba/GDN state slots, the
  linear-attention state is checkpointed next to the KV, and cached
  checkpoints are reused without mutation through copy-on-write.
* 24-ai.news TokenSpeed article, optimisation list, "hybrid prefix caching":
  the logical cache lives in C++ and the physical tensors in Python; radix
  matching with MambaSlot extensions reuses state with copy-on-write.

The pages give no allocation policy.  Bit-exact comparison with the C++
manager needs one fixed policy, so this model *is* that policy (a reading):

* Free list: an explicit list, initialised from a caller-supplied order (the
  caller draws the permutation; identity when none is given).  ``alloc`` pops
  from the END, ``free`` pushes to the END.
* Sequence ids: ``seq_create``/``seq_fork`` take the lowest unused id.
* ``fork(src, n)`` aliases the first ceil(n/P) pages of ``src`` (refcount+1
  each); the new sequence has length n.
* ``reserve(seq, n)``: if the last page is partially filled and shared
  (refcount > 1) it is copied first: a fresh page ``dst`` is popped, the
  triple (src, dst, valid = len % P) is reported, src loses one reference and
  dst replaces it.  Then whole pages are popped, in order, until the sequence
  covers len + n tokens.  The call is transactional: it checks capacity
  (``max_pages_per_seq``) and free pages first and changes nothing on error.
* ``truncate(seq, m)`` keeps ceil(m/P) pages, dropping the others from the
  last backwards; a page whose refcount reaches 0 is pushed on the free list
  at that moment.
* ``export`` pads page-table rows with -1.

Errors are raised as ``ModelError(kind)``; kinds: 'invalid', 'bad_seq',
'range', 'capacity', 'out_of_pages', 'out_of_slots', 'bad_slot'.
"""

import numpy as np


class ModelError(Exception):
    def __init__(self, kind):
        super().__init__(kind)
        self.kind = kind


def _ceil_div(a, b):
    return -(-a // b)


class PageTableModel:
    def __init__(self, num_pages, page_size, max_seqs, max_pages_per_seq, free_order=None):
        if num_pages <= 0 or page_size <= 0 or max_seqs <= 0 or max_pages_per_seq <= 0:
            raise ModelError("invalid")
        if free_order is None:
            free_order = list(range(num_pages))
        free_order = [int(p) for p in free_order]
        if sorted(free_order) != list(range(num_pages)):
            raise ModelError("invalid")
        self.num_pages = num_pages
        self.P = page_size
        self.max_seqs = max_seqs
        self.max_pages = max_pages_per_seq
        self.free = list(free_order)
        self.ref = [0] * num_pages
        self.seqs = {}

    # -- helpers ---------------------------------------------------------
    def _get(self, sid):
        if sid not in self.seqs:
            raise ModelError("bad_seq")
        return self.seqs[sid]

    def _new_id(self):
        for sid in range(self.max_seqs):
            if sid not in self.seqs:
                return sid
        raise ModelError("capacity")

    # -- operations ------------------------------------------------------
    def seq_create(self):
        sid = self._new_id()
        self.seqs[sid] = {"pages": [], "len": 0}
        return sid

    def seq_fork(self, src, prefix_len):
        s = self._get(src)
        if prefix_len < 0 or prefix_len > s["len"]:
            raise ModelError("range")
        sid = self._new_id()
        pages = s["pages"][: _ceil_div(prefix_len, self.P)]
        for p in pages:
            self.ref[p] += 1
        self.seqs[sid] = {"pages": list(pages), "len": prefix_len}
        return sid

    def reserve(self, sid, n):
        """Grow ``sid`` by n tokens; returns None or the CoW triple."""
        s = self._get(sid)
        if n < 0:
            raise ModelError("invalid")
        if n == 0:
            return None
        L, pages = s["len"], s["pages"]
        cow = (L % self.P != 0) and self.ref[pages[-1]] > 1
        need = _ceil_div(L + n, self.P) - len(pages)
        if len(pages) + need > self.max_pages:
            raise ModelError("capacity")
        if need + (1 if cow else 0) > len(self.free):
            raise ModelError("out_of_pages")
        triple = None
        if cow:
            src = pages[-1]
            dst = self.free.pop()
            self.ref[src] -= 1
            self.ref[dst] = 1
            pages[-1] = dst
            triple = (src, dst, L % self.P)
        for _ in range(need):
            p = self.free.pop()
            self.ref[p] = 1
            pages.append(p)
        s["len"] = L + n
        return triple

    def truncate(self, sid, m):
        s = self._get(sid)
        if m < 0 or m > s["len"]:
            raise ModelError("range")
        keep = _ceil_div(m, self.P)
        pages = s["pages"]
        while len(pages) > keep:
            p = pages.pop()
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)
        s["len"] = m

    def seq_free(self, sid):
        self.truncate(sid, 0)
        del self.seqs[sid]

    def export(self, sids, max_pages):
        pt = np.full((len(sids), max_pages), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, sid in enumerate(sids):
            s = self._get(sid)
            if len(s["pages"]) > max_pages:
                raise ModelError("invalid")
            pt[i, : len(s["pages"])] = s["pages"]
            lens[i] = s["len"]
        return pt, lens

    def stats(self):
        return len(self.free), sum(1 for r in self.ref if r > 0)


class SlotPoolModel:
    """Recurrent-state slot pool: refcounted slot ids, free list as above."""

    def __init__(self, n_slots, free_order=None):
        if n_slots <= 0:
            raise ModelError("invalid")
        if free_order is None:
            free_order = list(range(n_slots))
        free_order = [int(x) for x in free_order]
        if sorted(free_order) != list(range(n_slots)):
            raise ModelError("invalid")
        self.n = n_slots
        self.free = list(free_order)
        self.ref = [0] * n_slots

    def acquire(self):
        if not self.free:
            raise ModelError("out_of_slots")
        s = self.free.pop()
        self.ref[s] = 1
        return s

    def retain(self, s):
        if not (0 <= s < self.n) or self.ref[s] == 0:
            raise ModelError("bad_slot")
        self.ref[s] += 1

    def release(self, s):
        if not (0 <= s < self.n) or self.ref[s] == 0:
            raise ModelError("bad_slot")
        self.ref[s] -= 1
        if self.ref[s] == 0:
            self.free.append(s)

    def stats(self):
        return len(self.free), sum(1 for r in self.ref if r > 0)


def gather(pool, pages, seq_len, page_size, head=None):
    """Logical rows 0..seq_len-1 of one sequence, read through its pages.

    ``pool`` has layout [num_pages, H_kv, P, D]; position t lives at
    pool[pages[t // P], :, t % P, :].  Returns [seq_len, H_kv, D] (or
    [seq_len, D] when ``head`` is given) in the pool's own dtype, so a
    bf16-bits pool gathers bit-exactly.
    """
    t = np.arange(seq_len)
    phys = np.asarray(pages, dtype=np.int64)[t // page_size]
    off = t % page_size
    if head is None:
        return pool[phys, :, off, :]
    return pool[phys, head, off, :]


def scatter_contiguous(rows, pages, page_size, pool):
    """Inverse of ``gather``: write logical rows [L, H_kv, D] into ``pool``."""
    L = rows.shape[0]
    t = np.arange(L)
    phys = np.asarray(pages, dtype=np.int64)[t // page_size]
    pool[phys, :, t % page_size, :] = rows
    return pool
