"""Softmax decode attention over a paged context (fp64 definition).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* 24-ai.news TokenSpeed article: the served model is hybrid, standard
  full-attention layers interleaved with Gated DeltaNet layers (paragraph on
  the model architecture); contexts run to 1M tokens (long-context table);
  head dimension 256 (closing paragraph on FA4).
* zubnet.ai TokenSpeed article, second paragraph: the KV cache is paged, and
  speculative decoding is supported.

The attention itself is the textbook scaled dot-product softmax attention
(Vaswani et al., 2017) applied to one decode step.  Readings, since the pages
are silent:

* ``sm_scale`` is a parameter (1/sqrt(D) by default).
* Grouped-query attention groups consecutive query heads: query head hq uses
  KV head hq // G with G = H_q / H_kv.
* With q_len > 1 (draft tokens being verified), query j (0-based) sees the
  keys at positions < seq_len - q_len + j + 1: causal inside the draft.

``attention`` is the two-pass definition over the whole visible context; it
is neither online nor split.  ``split_partials`` and ``lse_merge`` state the
split-K decomposition (unnormalised partial output, running max, running
sum) so the combine step can be checked on its own.
"""

import numpy as np

from . import bf16
from .paging import gather


def attention(q, K, V, sm_scale):
    """q [q_len, H_q, D]; K, V [L, H_kv, D] (float64).  Returns [q_len, H_q, D]."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    q_len, H_q, D = q.shape
    L, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.empty((q_len, H_q, V.shape[2]), np.float64)
    for j in range(q_len):
        n = L - q_len + j + 1
        for h in range(H_kv):
            qs = q[j, h * G:(h + 1) * G, :]            # [G, D]
            x = sm_scale * (K[:n, h, :] @ qs.T)        # [n, G]
            p = np.exp(x - x.max(axis=0, keepdims=True))
            out[j, h * G:(h + 1) * G, :] = (p.T @ V[:n, h, :]) / p.sum(axis=0)[:, None]
    return out


def paged_attention(q_bits, k_pool_bits, v_pool_bits, page_table, seq_lens, page_size, sm_scale):
    """Batched decode attention read through the page table.

    q_bits [S, q_len, H_q, D] bf16 bits; pools [N, H_kv, P, D] bf16 bits;
    page_table [S, max_pages] int32; seq_lens [S] (lengths that include the
    q_len new tokens).  Returns float64 [S, q_len, H_q, D].
    """
    S = q_bits.shape[0]
    out = []
    for s in range(S):
        L = int(seq_lens[s])
        K = bf16.to_f64(gather(k_pool_bits, page_table[s], L, page_size))
        V = bf16.to_f64(gather(v_pool_bits, page_table[s], L, page_size))
        out.append(attention(bf16.to_f64(q_bits[s]), K, V, sm_scale))
    return np.stack(out)


def split_partials(q, K, V, sm_scale, bounds):
    """Per-split unnormalised partials for token ranges ``bounds`` [(t0, t1)].

    For each split, query j and head hq over the visible keys
    t in [t0, min(t1, n_j)):  m = max score (natural-log units), l = sum of
    exp(score - m), o = sum of exp(score - m) * v.  A split with no visible
    key has m = -inf, l = 0, o = 0.
    Returns o [n_split, q_len, H_q, D], m and l [n_split, q_len, H_q].
    """
    q = np.asarray(q, np.float64)
    q_len, H_q, D = q.shape
    L, H_kv, Dv = V.shape
    G = H_q // H_kv
    ns = len(bounds)
    o = np.zeros((ns, q_len, H_q, Dv))
    m = np.full((ns, q_len, H_q), -np.inf)
    l = np.zeros((ns, q_len, H_q))
    for si, (t0, t1) in enumerate(bounds):
        for j in range(q_len):
            n = L - q_len + j + 1
            hi = min(t1, n)
            if hi <= t0:
                continue
            for hq in range(H_q):
                h = hq // G
                x = sm_scale * (K[t0:hi, h, :] @ q[j, hq])
                mx = x.max()
                p = np.exp(x - mx)
                m[si, j, hq] = mx
                l[si, j, hq] = p.sum()
                o[si, j, hq] = p @ V[t0:hi, h, :]
    return o, m, l


def lse_merge(o_parts, m_parts, l_parts):
    """Merge split partials: o = sum_s w_s o_s / sum_s w_s l_s, w_s = exp(m_s - max m).

    Splits with m = -inf carry weight 0.  Returns [q_len, H_q, D].
    """
    m = np.max(m_parts, axis=0)
    w = np.where(np.isfinite(m_parts), np.exp(m_parts - m[None]), 0.0)
    num = np.sum(w[..., None] * o_parts, axis=0)
    den = np.sum(w * l_parts, axis=0)
    return num / den[..., None]
