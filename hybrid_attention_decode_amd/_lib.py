"""ctypes binding of libhad.so (argument marshalling only).

Every computation runs in the library: the host page-table/slot manager in
C++ and the decode path in gfx950 HIP kernels.  Device tensors are torch
tensors on a ROCm device; their data pointers and torch's current stream
are handed to the C ABI.  There is no fallback: if the library is missing,
every call raises.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhad.so")

OK = 0
_STATUS = {
    -1: "invalid",
    -2: "unsupported_shape",
    -3: "out_of_pages",
    -4: "out_of_slots",
    -5: "bad_seq",
    -6: "workspace_too_small",
    -7: "hip",
    -8: "bad_slot",
    -9: "capacity",
    -10: "range",
}
DERR_PAGE, DERR_SLOT, DERR_SEQLEN, DERR_COPY = 1, 2, 4, 8
ATTN_DETERMINISTIC = 1
ATTN_GATED_OUTPUT = 4
GDN_RAW_GATES = 1


class HadError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, status, message):
        self.status = status
        self.kind = _STATUS.get(status, "unknown")
        super().__init__("libhad status %d (%s): %s" % (status, self.kind, message))


_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)


class KvLayout(ctypes.Structure):
    _fields_ = [("num_pages", _i32), ("H_kv", _i32), ("page_size", _i32), ("head_dim", _i32)]


class QknrgDesc(ctypes.Structure):
    _fields_ = [("n_seqs", _i32), ("T", _i32), ("H_q", _i32), ("H_kv", _i32), ("head_dim", _i32),
                ("rotary_dim", _i32), ("rope_base", ctypes.c_double), ("eps", ctypes.c_float),
                ("num_pages", _i32), ("page_size", _i32), ("max_pages", _i32)]


class QknrgPtrs(ctypes.Structure):
    _fields_ = [("qg", _p), ("k", _p), ("v", _p), ("w_q", _p), ("w_k", _p), ("page_table", _p),
                ("seq_lens", _p), ("k_pool", _p), ("v_pool", _p), ("q_out", _p), ("gate_out", _p), ("d_err", _p)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n_seqs", _i32), ("q_len", _i32), ("H_q", _i32), ("H_kv", _i32), ("head_dim", _i32),
                ("num_pages", _i32), ("page_size", _i32), ("max_pages", _i32), ("sm_scale", ctypes.c_float),
                ("max_seq_len", _i32), ("num_splits", _i32), ("flags", _i32)]


class AttnPtrs(ctypes.Structure):
    _fields_ = [("q", _p), ("k_pool", _p), ("v_pool", _p), ("page_table", _p), ("seq_lens", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t), ("out", _p), ("d_err", _p), ("gate", _p)]


class AttnPrefix(ctypes.Structure):
    _fields_ = [("prefix_pages", _i32), ("prefix_page_table", _p)]


class GdnDesc(ctypes.Structure):
    _fields_ = [("n_seqs", _i32), ("T", _i32), ("H", _i32), ("d_k", _i32), ("d_v", _i32), ("n_slots", _i32),
                ("q_scale", ctypes.c_float), ("flags", _i32)]


class GdnPtrs(ctypes.Structure):
    _fields_ = [("state_pool", _p), ("in_idx", _p), ("out_idx", _p), ("q", _p), ("k", _p), ("v", _p),
                ("alpha", _p), ("beta", _p), ("o", _p), ("d_err", _p)]


class GdnPrefillDesc(ctypes.Structure):
    _fields_ = [("n_seqs", _i32), ("H", _i32), ("d_k", _i32), ("d_v", _i32), ("n_slots", _i32), ("max_len", _i32),
                ("q_scale", ctypes.c_float), ("flags", _i32), ("n_segments", _i32)]


class GdnPrefillPtrs(ctypes.Structure):
    _fields_ = [("state_pool", _p), ("in_idx", _p), ("out_idx", _p), ("cu_seqlens", _p), ("q", _p), ("k", _p),
                ("v", _p), ("alpha", _p), ("beta", _p), ("o", _p), ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t), ("d_err", _p)]


_SIGS = {
    "had_abi_version": ([], ctypes.c_int),
    "had_last_error": ([], ctypes.c_char_p),
    "had_kvpt_create": ([_i32, _i32, _i32, _i32, _pi32, ctypes.POINTER(_p)], ctypes.c_int),
    "had_kvpt_destroy": ([_p], ctypes.c_int),
    "had_kvpt_seq_create": ([_p, _pi32], ctypes.c_int),
    "had_kvpt_seq_fork": ([_p, _i32, _i32, _pi32], ctypes.c_int),
    "had_kvpt_reserve": ([_p, _i32, _i32, _pi32, _pi32], ctypes.c_int),
    "had_kvpt_truncate": ([_p, _i32, _i32], ctypes.c_int),
    "had_kvpt_seq_free": ([_p, _i32], ctypes.c_int),
    "had_kvpt_seq_len": ([_p, _i32, _pi32], ctypes.c_int),
    "had_kvpt_export": ([_p, _pi32, _i32, _pi32, _i32, _pi32], ctypes.c_int),
    "had_kvpt_stats": ([_p, _pi32, _pi32], ctypes.c_int),
    "had_kvpt_info": ([_p, _pi32, _pi32], ctypes.c_int),
    "had_kvpt_seq_create_from": ([_p, _pi32, _i32, _i32, _pi32], ctypes.c_int),
    "had_kvpt_page_retain": ([_p, _i32], ctypes.c_int),
    "had_kvpt_page_release": ([_p, _i32], ctypes.c_int),
    "had_radix_create": ([_p, _p, ctypes.POINTER(_p)], ctypes.c_int),
    "had_radix_destroy": ([_p], ctypes.c_int),
    "had_radix_match": ([_p, _pi32, _i32, _pi32, _pi32, _pi32, _i32, _pi32], ctypes.c_int),
    "had_radix_unlock": ([_p, _i32], ctypes.c_int),
    "had_radix_insert": ([_p, _pi32, _i32, _pi32, _i32, _pi32], ctypes.c_int),
    "had_radix_evict": ([_p, _i32, _i32, _pi32], ctypes.c_int),
    "had_radix_stats": ([_p, _pi32, ctypes.POINTER(ctypes.c_int64), _pi32, ctypes.POINTER(ctypes.c_int64),
                         ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
    "had_slots_create": ([_i32, _pi32, ctypes.POINTER(_p)], ctypes.c_int),
    "had_slots_destroy": ([_p], ctypes.c_int),
    "had_slots_acquire": ([_p, _pi32], ctypes.c_int),
    "had_slots_retain": ([_p, _i32], ctypes.c_int),
    "had_slots_release": ([_p, _i32], ctypes.c_int),
    "had_slots_stats": ([_p, _pi32, _pi32], ctypes.c_int),
    "had_spec_rollback": ([_p, _p, _i32, _i32, _i32, _i32, _pi32, _pi32], ctypes.c_int),
    "had_kv_copy_pages": ([ctypes.POINTER(KvLayout), _p, _p, _p, _p, _i32, _p, _p], ctypes.c_int),
    "had_kv_check_copy_pages": ([_i32, _pi32, _pi32, _i32], ctypes.c_int),
    "had_attn_check_prefix": ([_i32, _i32, _pi32, _i32, _pi32], ctypes.c_int),
    "had_kv_append": ([ctypes.POINTER(KvLayout), _p, _p, _p, _i32, _p, _p, _p, _i32, _i32, _p, _p], ctypes.c_int),
    "had_qk_norm_rope_gate": ([ctypes.POINTER(QknrgDesc), ctypes.POINTER(QknrgPtrs), _p], ctypes.c_int),
    "had_decode_attn_plan": ([ctypes.POINTER(AttnDesc), _pi32, _pi32], ctypes.c_int),
    "had_decode_attn_workspace_bytes": ([ctypes.POINTER(AttnDesc)], ctypes.c_size_t),
    "had_decode_attn": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPtrs), _p], ctypes.c_int),
    "had_decode_attn_partial": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPtrs), _p], ctypes.c_int),
    "had_decode_attn_combine": ([ctypes.POINTER(AttnDesc), _i32, _p, _p, _p], ctypes.c_int),
    "had_decode_attn_cascade_workspace_bytes": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPrefix)],
                                                ctypes.c_size_t),
    "had_decode_attn_cascade": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPrefix), ctypes.POINTER(AttnPtrs), _p],
                                ctypes.c_int),
    "had_decode_attn_cascade_plan": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPrefix), _pi32, _pi32],
                                     ctypes.c_int),
    "had_decode_attn_cascade_partial": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPrefix),
                                        ctypes.POINTER(AttnPtrs), _i32, _p], ctypes.c_int),
    "had_decode_attn_cascade_combine": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnPrefix),
                                        ctypes.POINTER(AttnPtrs), _p], ctypes.c_int),
    "had_decode_attn_layer": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(QknrgDesc), ctypes.POINTER(QknrgPtrs), _p,
                               ctypes.c_size_t, _p, _p], ctypes.c_int),
    "had_decode_attn_layer_static": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(QknrgDesc), ctypes.POINTER(QknrgPtrs),
                                      _p, _p], ctypes.c_int),
    "had_decode_attn_layer_partial": ([ctypes.POINTER(AttnDesc), ctypes.POINTER(QknrgDesc),
                                       ctypes.POINTER(QknrgPtrs), _p, ctypes.c_size_t, _p], ctypes.c_int),
    "had_gdn_state_update": ([ctypes.POINTER(GdnDesc), ctypes.POINTER(GdnPtrs), _p], ctypes.c_int),
    "had_gdn_check_slots": ([_i32, _i32, _i32, _pi32, _pi32, _i32], ctypes.c_int),
    "had_gdn_prefill_workspace_bytes": ([ctypes.POINTER(GdnPrefillDesc)], ctypes.c_size_t),
    "had_gdn_prefill": ([ctypes.POINTER(GdnPrefillDesc), ctypes.POINTER(GdnPrefillPtrs), _p], ctypes.c_int),
}

_lib = None


def lib():
    """Load libhad.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhad.so is not built (%s); run `python -m hybrid_attention_decode_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _check(status):
    if status != OK:
        raise HadError(status, lib().had_last_error().decode(errors="replace"))


def abi_version():
    return lib().had_abi_version()


def _i32_array(values):
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data_as(_pi32)


# ----------------------------------------------------------------- host side

class PageTable:
    """Handle on the C++ page-table manager (had_kvpt_*)."""

    def __init__(self, num_pages, page_size, max_seqs, max_pages_per_seq, free_order=None):
        self._h = _p()
        if free_order is not None:
            self._order, ptr = _i32_array(free_order)
        else:
            ptr = None
        _check(lib().had_kvpt_create(num_pages, page_size, max_seqs, max_pages_per_seq, ptr, ctypes.byref(self._h)))
        self.page_size = page_size

    def close(self):
        if self._h:
            lib().had_kvpt_destroy(self._h)
            self._h = _p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_create(self):
        out = _i32()
        _check(lib().had_kvpt_seq_create(self._h, ctypes.byref(out)))
        return out.value

    def seq_fork(self, src, prefix_len):
        out = _i32()
        _check(lib().had_kvpt_seq_fork(self._h, src, prefix_len, ctypes.byref(out)))
        return out.value

    def reserve(self, seq, n_tokens):
        """Returns None or the copy-on-write triple (src, dst, valid)."""
        cow = (_i32 * 3)()
        n = _i32()
        _check(lib().had_kvpt_reserve(self._h, seq, n_tokens, cow, ctypes.byref(n)))
        return (cow[0], cow[1], cow[2]) if n.value else None

    def truncate(self, seq, new_len):
        _check(lib().had_kvpt_truncate(self._h, seq, new_len))

    def seq_free(self, seq):
        _check(lib().had_kvpt_seq_free(self._h, seq))

    def seq_len(self, seq):
        out = _i32()
        _check(lib().had_kvpt_seq_len(self._h, seq, ctypes.byref(out)))
        return out.value

    def export(self, seqs, max_pages):
        seqs_a, sp = _i32_array(seqs)
        n = len(seqs_a)
        table = np.zeros((n, max_pages), dtype=np.int32)
        lens = np.zeros(n, dtype=np.int32)
        _check(lib().had_kvpt_export(self._h, sp, n, table.ctypes.data_as(_pi32), max_pages,
                                     lens.ctypes.data_as(_pi32)))
        return table, lens

    def stats(self):
        f, u = _i32(), _i32()
        _check(lib().had_kvpt_stats(self._h, ctypes.byref(f), ctypes.byref(u)))
        return f.value, u.value

    def info(self):
        n, ps = _i32(), _i32()
        _check(lib().had_kvpt_info(self._h, ctypes.byref(n), ctypes.byref(ps)))
        return n.value, ps.value

    def seq_create_from(self, pages, length):
        arr, ptr = _i32_array(pages)
        out = _i32()
        _check(lib().had_kvpt_seq_create_from(self._h, ptr, len(arr), length, ctypes.byref(out)))
        return out.value

    def page_retain(self, page):
        _check(lib().had_kvpt_page_retain(self._h, page))

    def page_release(self, page):
        _check(lib().had_kvpt_page_release(self._h, page))


class SlotPool:
    """Handle on the C++ state-slot pool (had_slots_*)."""

    def __init__(self, n_slots, free_order=None):
        self._h = _p()
        if free_order is not None:
            self._order, ptr = _i32_array(free_order)
        else:
            ptr = None
        _check(lib().had_slots_create(n_slots, ptr, ctypes.byref(self._h)))

    def close(self):
        if self._h:
            lib().had_slots_destroy(self._h)
            self._h = _p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def acquire(self):
        out = _i32()
        _check(lib().had_slots_acquire(self._h, ctypes.byref(out)))
        return out.value

    def retain(self, slot):
        _check(lib().had_slots_retain(self._h, slot))

    def release(self, slot):
        _check(lib().had_slots_release(self._h, slot))

    def stats(self):
        f, u = _i32(), _i32()
        _check(lib().had_slots_stats(self._h, ctypes.byref(f), ctypes.byref(u)))
        return f.value, u.value


class RadixCache:
    """Hybrid prefix cache (had_radix_*): a radix tree over token ids whose
    nodes hold KV pages and, where a state was saved, a GDN state slot.
    Works on a PageTable and a SlotPool, which must outlive it."""

    def __init__(self, pt, slots):
        self._pt, self._slots = pt, slots  # keep the pools alive while the cache holds references
        self._h = _p()
        _check(lib().had_radix_create(pt._h, slots._h, ctypes.byref(self._h)))
        self.page_size = pt.info()[1]

    def close(self):
        if self._h:
            lib().had_radix_destroy(self._h)
            self._h = _p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def match(self, tokens):
        """Returns (matched_len, slot, pages, lock)."""
        arr, ptr = _i32_array(tokens)
        maxp = -(-len(arr) // self.page_size)
        pages = np.full(max(maxp, 1), -1, dtype=np.int32)
        m, sl, lk = _i32(), _i32(), _i32()
        _check(lib().had_radix_match(self._h, ptr, len(arr), ctypes.byref(m), ctypes.byref(sl),
                                     pages.ctypes.data_as(_pi32), len(pages), ctypes.byref(lk)))
        return m.value, sl.value, pages[:-(-m.value // self.page_size)].tolist(), lk.value

    def unlock(self, lock):
        _check(lib().had_radix_unlock(self._h, lock))

    def insert(self, tokens, pages, slot):
        """Returns the number of tokens not cached before."""
        arr, ptr = _i32_array(tokens)
        parr, pptr = _i32_array(pages)
        if len(parr) != -(-len(arr) // self.page_size):
            raise ValueError("insert: %d pages for %d tokens" % (len(parr), len(arr)))
        nt = _i32()
        _check(lib().had_radix_insert(self._h, ptr, len(arr), pptr, slot, ctypes.byref(nt)))
        return nt.value

    def evict(self, min_free_pages, min_free_slots=0):
        n = _i32()
        _check(lib().had_radix_evict(self._h, min_free_pages, min_free_slots, ctypes.byref(n)))
        return n.value

    def stats(self):
        nn, nc = _i32(), _i32()
        toks, q, m = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().had_radix_stats(self._h, ctypes.byref(nn), ctypes.byref(toks), ctypes.byref(nc),
                                     ctypes.byref(q), ctypes.byref(m)))
        return dict(nodes=nn.value, cached_tokens=toks.value, checkpoints=nc.value, queried_tokens=q.value,
                    matched_tokens=m.value)


def spec_rollback(pt, slots, seq, T, accepted, in_slot, out_slots):
    outs, op = _i32_array(out_slots)
    cur = _i32()
    _check(lib().had_spec_rollback(pt._h, slots._h, seq, T, accepted, in_slot, op, ctypes.byref(cur)))
    return cur.value


# --------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def _stream():
    return _p(_torch().cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return _p(t.data_ptr())


def _opt(t, name):
    return None if t is None else _dev(t, _torch().int32, name)


def kv_check_copy_pages(num_pages, src, dst):
    """Host check of a page-copy list (see had_kv_check_copy_pages); src, dst
    as host sequences or tensors.  Raises HadError."""
    if hasattr(src, "cpu"):
        src, dst = src.cpu().numpy(), dst.cpu().numpy()
    s_a, sp = _i32_array(np.asarray(src).reshape(-1))
    d_a, dp = _i32_array(np.asarray(dst).reshape(-1))
    if len(s_a) != len(d_a):
        raise ValueError("src and dst differ in length")
    _check(lib().had_kv_check_copy_pages(int(num_pages), sp, dp, len(s_a)))


def kv_copy_pages(k_pool, v_pool, src, dst, d_err=None):
    """Copy whole pages src[i] -> dst[i] in both pools.  src, dst: int32 device
    tensors (read when the copy runs; a -1 source marks an unused entry) or
    host sequences (copied to the device first)."""
    torch = _torch()
    N, H_kv, P, D = k_pool.shape
    L = KvLayout(N, H_kv, P, D)
    if not isinstance(src, torch.Tensor):
        src = torch.tensor(np.asarray(src, dtype=np.int32).reshape(-1), device=k_pool.device)
    if not isinstance(dst, torch.Tensor):
        dst = torch.tensor(np.asarray(dst, dtype=np.int32).reshape(-1), device=k_pool.device)
    if src.numel() != dst.numel():
        raise ValueError("src and dst differ in length")
    if _debug():
        kv_check_copy_pages(N, src, dst)
    _check(lib().had_kv_copy_pages(ctypes.byref(L), _dev(k_pool, torch.bfloat16, "k_pool"),
                                   _dev(v_pool, torch.bfloat16, "v_pool"), _dev(src, torch.int32, "src"),
                                   _dev(dst, torch.int32, "dst"), src.numel(), _opt(d_err, "d_err"), _stream()))


def attn_check_prefix(page_table, prefix_page_table):
    """Host check of the cascade precondition (see had_attn_check_prefix):
    every row of page_table [S, max_pages] begins with prefix_page_table.
    Host arrays or tensors.  Raises HadError."""
    if hasattr(page_table, "cpu"):
        page_table = page_table.cpu().numpy()
    if hasattr(prefix_page_table, "cpu"):
        prefix_page_table = prefix_page_table.cpu().numpy()
    pt = np.asarray(page_table, dtype=np.int32)
    pa, pp = _i32_array(pt)
    xa, xp = _i32_array(np.asarray(prefix_page_table).reshape(-1))
    _check(lib().had_attn_check_prefix(pa.shape[0], pa.shape[1], pp, len(xa), xp))


def kv_append(k_pool, v_pool, page_table, seq_lens, k_new, v_new, d_err=None):
    torch = _torch()
    N, H_kv, P, D = k_pool.shape
    n_seqs, t_new = k_new.shape[0], k_new.shape[1]
    L = KvLayout(N, H_kv, P, D)
    _check(lib().had_kv_append(ctypes.byref(L), _dev(k_pool, torch.bfloat16, "k_pool"),
                               _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                               page_table.shape[1], _dev(seq_lens, torch.int32, "seq_lens"),
                               _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
                               n_seqs, t_new, _opt(d_err, "d_err"), _stream()))


def qk_norm_rope_gate(qg, k, v, w_q, w_k, page_table, seq_lens, k_pool, v_pool, rotary_dim,
                      rope_base=10000.0, eps=1e-6, q_out=None, gate_out=None, d_err=None):
    """qg [S, T, H_q, 2, D], k/v [S, T, H_kv, D] -> (q_out, gate_out) [S, T, H_q, D]."""
    torch = _torch()
    S, T, H_q, two, D = qg.shape
    H_kv = k.shape[2]
    if q_out is None:
        q_out = torch.empty((S, T, H_q, D), dtype=torch.bfloat16, device=qg.device)
    if gate_out is None:
        gate_out = torch.empty((S, T, H_q, D), dtype=torch.bfloat16, device=qg.device)
    desc = QknrgDesc(S, T, H_q, H_kv, D, rotary_dim, float(rope_base), float(eps), k_pool.shape[0],
                     k_pool.shape[2], page_table.shape[1])
    ptrs = QknrgPtrs(_dev(qg, torch.bfloat16, "qg"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                     _dev(w_q, torch.float32, "w_q"), _dev(w_k, torch.float32, "w_k"),
                     _dev(page_table, torch.int32, "page_table"), _dev(seq_lens, torch.int32, "seq_lens"),
                     _dev(k_pool, torch.bfloat16, "k_pool"), _dev(v_pool, torch.bfloat16, "v_pool"),
                     _dev(q_out, torch.bfloat16, "q_out"), _dev(gate_out, torch.bfloat16, "gate_out"),
                     _opt(d_err, "d_err"))
    _check(lib().had_qk_norm_rope_gate(ctypes.byref(desc), ctypes.byref(ptrs), _stream()))
    return q_out, gate_out


def attn_desc(q_shape, k_pool_shape, max_pages, sm_scale=None, max_seq_len=0, num_splits=0, deterministic=False,
              gated=False):
    S, q_len, H_q, D = q_shape
    N, H_kv, P, D2 = k_pool_shape
    if D != D2:
        raise ValueError("q and pool head_dim differ")
    if sm_scale is None:
        sm_scale = 1.0 / float(np.sqrt(D))
    return AttnDesc(S, q_len, H_q, H_kv, D, N, P, max_pages, float(sm_scale), int(max_seq_len), int(num_splits),
                    (ATTN_DETERMINISTIC if deterministic else 0) | (ATTN_GATED_OUTPUT if gated else 0))


def decode_attn_plan(desc):
    ns, pps = _i32(), _i32()
    _check(lib().had_decode_attn_plan(ctypes.byref(desc), ctypes.byref(ns), ctypes.byref(pps)))
    return ns.value, pps.value


def decode_attn_workspace_bytes(desc):
    n = lib().had_decode_attn_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        # the call reports an invalid descriptor by returning 0: surface why
        _check(lib().had_decode_attn_plan(ctypes.byref(desc), ctypes.byref(_i32()), ctypes.byref(_i32())))
    return n


def decode_attn(q, k_pool, v_pool, page_table, seq_lens, sm_scale=None, max_seq_len=0, num_splits=0,
                workspace=None, out=None, d_err=None, deterministic=False, gate=None):
    """q [S, q_len, H_q, D] bf16 -> out [S, q_len, H_q, D] bf16.
    gate (same shape, bf16): when given, out is multiplied by sigmoid(gate)."""
    torch = _torch()
    desc = attn_desc(q.shape, k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, num_splits, deterministic,
                     gate is not None)
    need = decode_attn_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ptrs = AttnPtrs(_dev(q, torch.bfloat16, "q"), _dev(k_pool, torch.bfloat16, "k_pool"),
                    _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                    _dev(seq_lens, torch.int32, "seq_lens"), _dev(workspace, torch.uint8, "workspace"),
                    workspace.numel(), _dev(out, torch.bfloat16, "out"), _opt(d_err, "d_err"),
                    None if gate is None else _dev(gate, torch.bfloat16, "gate"))
    _check(lib().had_decode_attn(ctypes.byref(desc), ctypes.byref(ptrs), _stream()))
    return out


def decode_attn_cascade(q, k_pool, v_pool, page_table, seq_lens, prefix_page_table, sm_scale=None, max_seq_len=0,
                        workspace=None, out=None, d_err=None, deterministic=False, gate=None):
    """Decode attention for a batch whose sequences share their first
    len(prefix_page_table) pages (read once for every sequence's rows).
    q [S, q_len, H_q, D] bf16; prefix_page_table int32 [prefix_pages] on the device.
    gate (like q): when given, out is multiplied by sigmoid(gate)."""
    torch = _torch()
    desc = attn_desc(q.shape, k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, 0, deterministic,
                     gate is not None)
    px = AttnPrefix(prefix_page_table.numel(), _dev(prefix_page_table, torch.int32, "prefix_page_table"))
    if _debug():
        attn_check_prefix(page_table, prefix_page_table)
    need = lib().had_decode_attn_cascade_workspace_bytes(ctypes.byref(desc), ctypes.byref(px))
    if need == 0:  # invalid descriptor or prefix: the call itself reports why
        _check(lib().had_decode_attn_cascade(ctypes.byref(desc), ctypes.byref(px), None, _stream()))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ptrs = AttnPtrs(_dev(q, torch.bfloat16, "q"), _dev(k_pool, torch.bfloat16, "k_pool"),
                    _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                    _dev(seq_lens, torch.int32, "seq_lens"), _dev(workspace, torch.uint8, "workspace"),
                    workspace.numel(), _dev(out, torch.bfloat16, "out"), _opt(d_err, "d_err"),
                    None if gate is None else _dev(gate, torch.bfloat16, "gate"))
    _check(lib().had_decode_attn_cascade(ctypes.byref(desc), ctypes.byref(px), ctypes.byref(ptrs), _stream()))
    return out


def decode_attn_cascade_plan(desc, prefix_pages):
    """(prefix_splits, suffix_splits) of the cascade's plan."""
    px = AttnPrefix(prefix_pages, None)
    a, b = _i32(), _i32()
    _check(lib().had_decode_attn_cascade_plan(ctypes.byref(desc), ctypes.byref(px), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def decode_attn_cascade_partial(q, k_pool, v_pool, page_table, seq_lens, prefix_page_table, workspace, passes,
                                sm_scale=None, max_seq_len=0, d_err=None, deterministic=False):
    """The cascade's prefix pass (passes = 1), suffix pass (2) or both (3),
    partials only; decode_attn_cascade_combine finishes."""
    torch = _torch()
    desc = attn_desc(q.shape, k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, 0, deterministic, False)
    px = AttnPrefix(prefix_page_table.numel(), _dev(prefix_page_table, torch.int32, "prefix_page_table"))
    ptrs = AttnPtrs(_dev(q, torch.bfloat16, "q"), _dev(k_pool, torch.bfloat16, "k_pool"),
                    _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                    _dev(seq_lens, torch.int32, "seq_lens"), _dev(workspace, torch.uint8, "workspace"),
                    workspace.numel(), None, _opt(d_err, "d_err"), None)
    _check(lib().had_decode_attn_cascade_partial(ctypes.byref(desc), ctypes.byref(px), ctypes.byref(ptrs),
                                                 int(passes), _stream()))


def decode_attn_cascade_combine(q, k_pool, v_pool, page_table, seq_lens, prefix_page_table, workspace, out=None,
                                sm_scale=None, max_seq_len=0, d_err=None, deterministic=False, gate=None):
    """The cascade's merge of the partials decode_attn_cascade_partial wrote."""
    torch = _torch()
    desc = attn_desc(q.shape, k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, 0, deterministic,
                     gate is not None)
    px = AttnPrefix(prefix_page_table.numel(), _dev(prefix_page_table, torch.int32, "prefix_page_table"))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ptrs = AttnPtrs(_dev(q, torch.bfloat16, "q"), _dev(k_pool, torch.bfloat16, "k_pool"),
                    _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                    _dev(seq_lens, torch.int32, "seq_lens"), _dev(workspace, torch.uint8, "workspace"),
                    workspace.numel(), _dev(out, torch.bfloat16, "out"), _opt(d_err, "d_err"),
                    None if gate is None else _dev(gate, torch.bfloat16, "gate"))
    _check(lib().had_decode_attn_cascade_combine(ctypes.byref(desc), ctypes.byref(px), ctypes.byref(ptrs), _stream()))
    return out


def decode_attn_cascade_workspace_bytes(desc, prefix_pages):
    px = AttnPrefix(prefix_pages, None)
    return lib().had_decode_attn_cascade_workspace_bytes(ctypes.byref(desc), ctypes.byref(px))


def decode_attn_layer(qg, k, v, w_q, w_k, page_table, seq_lens, k_pool, v_pool, rotary_dim, rope_base=10000.0,
                      eps=1e-6, sm_scale=None, max_seq_len=0, num_splits=0, workspace=None, out=None, gate_out=None,
                      q_out=None, d_err=None, deterministic=False, partial_only=False, gated=False):
    """qk_norm_rope_gate + decode_attn in one pass (the prologue runs inside
    the attention kernel).  qg [S, T, H_q, 2, D]; k, v [S, T, H_kv, D].
    Returns (out, gate_out) [S, T, H_q, D]; q_out is written when given.
    partial_only: stop after the partials (workspace), out is not written.
    gated: out is multiplied by sigmoid(gate) before its rounding."""
    torch = _torch()
    S, T, H_q, two, D = qg.shape
    H_kv = k.shape[2]
    desc = attn_desc((S, T, H_q, D), k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, num_splits,
                     deterministic, gated)
    pdesc = QknrgDesc(S, T, H_q, H_kv, D, rotary_dim, float(rope_base), float(eps), k_pool.shape[0], k_pool.shape[2],
                      page_table.shape[1])
    need = decode_attn_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qg.device)
    if out is None:
        out = torch.empty((S, T, H_q, D), dtype=torch.bfloat16, device=qg.device)
    if gate_out is None:
        gate_out = torch.empty((S, T, H_q, D), dtype=torch.bfloat16, device=qg.device)
    ptrs = QknrgPtrs(_dev(qg, torch.bfloat16, "qg"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                     _dev(w_q, torch.float32, "w_q"), _dev(w_k, torch.float32, "w_k"),
                     _dev(page_table, torch.int32, "page_table"), _dev(seq_lens, torch.int32, "seq_lens"),
                     _dev(k_pool, torch.bfloat16, "k_pool"), _dev(v_pool, torch.bfloat16, "v_pool"),
                     None if q_out is None else _dev(q_out, torch.bfloat16, "q_out"),
                     _dev(gate_out, torch.bfloat16, "gate_out"), _opt(d_err, "d_err"))
    if partial_only:
        _check(lib().had_decode_attn_layer_partial(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(ptrs),
                                                   _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                                   _stream()))
    else:
        _check(lib().had_decode_attn_layer(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(ptrs),
                                           _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                           _dev(out, torch.bfloat16, "out"), _stream()))
    return out, gate_out


def decode_attn_layer_static(qg, k, v, w_q, w_k, page_table, seq_lens, k_pool, v_pool, rotary_dim, out, gate_out,
                             rope_base=10000.0, eps=1e-6, sm_scale=None, max_seq_len=0, num_splits=0, q_out=None,
                             d_err=None, deterministic=False, gated=False):
    """decode_attn_layer without a workspace argument and without any device
    allocation: the library's per-GPU static workspace is used (calls that
    overlap on one GPU race on it).  out and gate_out [S, T, H_q, D] bf16 are
    the caller's."""
    torch = _torch()
    S, T, H_q, two, D = qg.shape
    H_kv = k.shape[2]
    desc = attn_desc((S, T, H_q, D), k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, num_splits,
                     deterministic, gated)
    pdesc = QknrgDesc(S, T, H_q, H_kv, D, rotary_dim, float(rope_base), float(eps), k_pool.shape[0], k_pool.shape[2],
                      page_table.shape[1])
    ptrs = QknrgPtrs(_dev(qg, torch.bfloat16, "qg"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                     _dev(w_q, torch.float32, "w_q"), _dev(w_k, torch.float32, "w_k"),
                     _dev(page_table, torch.int32, "page_table"), _dev(seq_lens, torch.int32, "seq_lens"),
                     _dev(k_pool, torch.bfloat16, "k_pool"), _dev(v_pool, torch.bfloat16, "v_pool"),
                     None if q_out is None else _dev(q_out, torch.bfloat16, "q_out"),
                     _dev(gate_out, torch.bfloat16, "gate_out"), _opt(d_err, "d_err"))
    _check(lib().had_decode_attn_layer_static(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(ptrs),
                                              _dev(out, torch.bfloat16, "out"), _stream()))
    return out, gate_out


def decode_attn_partial(q, k_pool, v_pool, page_table, seq_lens, workspace, sm_scale=None, max_seq_len=0,
                        num_splits=0, d_err=None, deterministic=False):
    """Split-K partial kernel only: writes (o, m, l) partials to ``workspace``.
    Returns the descriptor (for decode_attn_combine)."""
    torch = _torch()
    desc = attn_desc(q.shape, k_pool.shape, page_table.shape[1], sm_scale, max_seq_len, num_splits, deterministic)
    ptrs = AttnPtrs(_dev(q, torch.bfloat16, "q"), _dev(k_pool, torch.bfloat16, "k_pool"),
                    _dev(v_pool, torch.bfloat16, "v_pool"), _dev(page_table, torch.int32, "page_table"),
                    _dev(seq_lens, torch.int32, "seq_lens"), _dev(workspace, torch.uint8, "workspace"),
                    workspace.numel(), None, _opt(d_err, "d_err"))
    _check(lib().had_decode_attn_partial(ctypes.byref(desc), ctypes.byref(ptrs), _stream()))
    return desc


def decode_attn_combine(desc, num_splits, workspace, out):
    torch = _torch()
    _check(lib().had_decode_attn_combine(ctypes.byref(desc), num_splits, _dev(workspace, workspace.dtype, "workspace"),
                                         _dev(out, torch.bfloat16, "out"), _stream()))
    return out


def gdn_check_slots(n_slots, in_idx, out_idx, allow_in_place):
    """Host check of the GDN slot preconditions (see had_gdn_check_slots);
    in_idx [S], out_idx [S, T] as host arrays or tensors.  Raises HadError."""
    if hasattr(in_idx, "cpu"):
        in_idx, out_idx = in_idx.cpu().numpy(), out_idx.cpu().numpy()
    ia, ip = _i32_array(np.asarray(in_idx).reshape(-1))
    oa = np.asarray(out_idx, dtype=np.int32).reshape(len(ia), -1)
    oa, op = _i32_array(oa)
    _check(lib().had_gdn_check_slots(len(ia), oa.shape[1] if oa.ndim == 2 else 1, int(n_slots), ip, op,
                                     1 if allow_in_place else 0))


def _debug():
    return os.environ.get("HAD_DEBUG") == "1"


def gdn_state_update(state_pool, in_idx, out_idx, q, k, v, alpha, beta, o=None, q_scale=1.0, d_err=None,
                     raw_gates=False):
    """state_pool [n_slots, H, d_v, d_k] fp32; q, k [S, T, H, d_k]; v [S, T, H, d_v] bf16;
    alpha, beta [S, T, H] fp32; in_idx [S], out_idx [S, T] int32 -> o [S, T, H, d_v] fp32.
    raw_gates: alpha, beta hold g and b; the kernel uses exp(g) and sigmoid(b)."""
    torch = _torch()
    n_slots, H, d_v, d_k = state_pool.shape
    S, T = out_idx.shape
    if o is None:
        o = torch.empty((S, T, H, d_v), dtype=torch.float32, device=state_pool.device)
    if _debug():
        gdn_check_slots(n_slots, in_idx, out_idx, T == 1)
    desc = GdnDesc(S, T, H, d_k, d_v, n_slots, float(q_scale), GDN_RAW_GATES if raw_gates else 0)
    ptrs = GdnPtrs(_dev(state_pool, torch.float32, "state_pool"), _dev(in_idx, torch.int32, "in_idx"),
                   _dev(out_idx, torch.int32, "out_idx"), _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"),
                   _dev(v, torch.bfloat16, "v"), _dev(alpha, torch.float32, "alpha"),
                   _dev(beta, torch.float32, "beta"), _dev(o, torch.float32, "o"), _opt(d_err, "d_err"))
    _check(lib().had_gdn_state_update(ctypes.byref(desc), ctypes.byref(ptrs), _stream()))
    return o


def gdn_prefill_desc(state_shape, n_seqs, max_len, q_scale=1.0, raw_gates=False, n_segments=0):
    n_slots, H, d_v, d_k = state_shape
    return GdnPrefillDesc(n_seqs, H, d_k, d_v, n_slots, int(max_len), float(q_scale),
                          GDN_RAW_GATES if raw_gates else 0, int(n_segments))


def gdn_prefill_workspace_bytes(desc):
    n = lib().had_gdn_prefill_workspace_bytes(ctypes.byref(desc))
    if n == 0 and desc.max_len > 0:
        _check(lib().had_gdn_prefill(ctypes.byref(desc), None, None))  # reports why the descriptor is invalid
    return n


def gdn_prefill(state_pool, in_idx, out_idx, cu_seqlens, q, k, v, alpha, beta, max_len=None, o=None, q_scale=1.0,
                workspace=None, d_err=None, raw_gates=False, n_segments=0):
    """Whole prompts through the gated delta rule, chunk-parallel.
    state_pool [n_slots, H, d_v, d_k] fp32; q, k [N, H, d_k], v [N, H, d_v] bf16 (sequences packed,
    token offsets cu_seqlens int32 [n_seqs + 1] on the device); alpha, beta [N, H] fp32;
    in_idx, out_idx int32 [n_seqs].  max_len bounds every sequence's length; the
    workspace holds n_seqs x ceil(max_len / 64) chunk blocks.  Default: the
    longest sequence, read from cu_seqlens (a device-to-host copy; pass
    max_len to avoid it, e.g. under graph capture).  n_segments: scan
    segments (0 = the library's choice; see had.h).
    Returns o [N, H, d_v] fp32; the final states land in slots out_idx."""
    torch = _torch()
    N, H, d_k = q.shape
    n_seqs = cu_seqlens.numel() - 1
    if max_len is None:
        if torch.cuda.is_current_stream_capturing():
            raise ValueError("gdn_prefill: pass max_len under graph capture (the default reads cu_seqlens to the host)")
        cu = cu_seqlens.cpu().numpy().astype(np.int64)
        max_len = int(max(1, (cu[1:] - cu[:-1]).max(initial=0)))
    if _debug():
        gdn_check_slots(state_pool.shape[0], in_idx, out_idx.reshape(-1, 1), True)
    desc = gdn_prefill_desc(state_pool.shape, n_seqs, max_len, q_scale, raw_gates, n_segments)
    need = gdn_prefill_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((N, H, state_pool.shape[2]), dtype=torch.float32, device=q.device)
    ptrs = GdnPrefillPtrs(_dev(state_pool, torch.float32, "state_pool"), _dev(in_idx, torch.int32, "in_idx"),
                          _dev(out_idx, torch.int32, "out_idx"), _dev(cu_seqlens, torch.int32, "cu_seqlens"),
                          _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
                          _dev(alpha, torch.float32, "alpha"), _dev(beta, torch.float32, "beta"),
                          _dev(o, torch.float32, "o"), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                          _opt(d_err, "d_err"))
    _check(lib().had_gdn_prefill(ctypes.byref(desc), ctypes.byref(ptrs), _stream()))
    return o
