"""QK-RMSNorm + partial rotary embedding + gate split (fp64 definition).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* zubnet.ai TokenSpeed article (Spanish and French), second paragraph: the
  engine fuses QK-RMSNorm, partial RoPE and the gate split into one kernel
  whose intermediates stay in registers.
* The agentic workload's per-layer shape (8 query heads, 1 KV head, head
  dimension 256, rotary embedding on 64 of the 256 dims) comes with the
  workload description; the pages' FA4 paragraph fixes head_dim 256.

The three steps are textbook operations:
* RMSNorm (Zhang & Sennrich, 2019): y = x / sqrt(mean(x**2) + eps) * w.
* Rotary position embedding (Su et al., RoFormer, 2021) applied to the first
  R dims only, with the "rotate-half" pairing (i, i + R/2), angle
  theta_i = pos * base**(-2i/R), i < R/2.
* Gate split: the projection output of each query head holds q then gate.
* Output gate: the attention output of a head is multiplied elementwise by
  sigmoid(gate) (the gated attention output of the full-attention layers).

Readings (pages silent): norm before rotation (the order of the name); the
first R dims rotate and the rest pass through; base 10000 and eps 1e-6 by
default; ``w`` is the final multiplier; qg layout [T, H_q, 2, D]; positions
of the T new tokens are seq_len_before + j; v is passed through unchanged;
the gate the split produces is applied as sigmoid(gate) * attention output,
per element of the head (the pages name the split, not where the gate acts).
Angles are computed in float64.
"""

import numpy as np


def rmsnorm(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope_partial(y, positions, rotary_dim, base):
    """Rotate the first ``rotary_dim`` dims of y [T, H, D] at positions [T]."""
    y = np.array(y, np.float64, copy=True)
    half = rotary_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / rotary_dim)
    theta = np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]   # [T, half]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    a = y[..., :half].copy()
    b = y[..., half:rotary_dim].copy()
    y[..., :half] = a * c - b * s
    y[..., half:rotary_dim] = b * c + a * s
    return y


def qk_norm_rope_gate(qg, k, v, w_q, w_k, positions, rotary_dim, base=10000.0, eps=1e-6):
    """One sequence's T new tokens.

    qg [T, H_q, 2, D], k and v [T, H_kv, D] (float64 values of the bf16
    inputs).  Returns (q_out [T, H_q, D], gate [T, H_q, D], k_out, v_out).
    """
    qg = np.asarray(qg, np.float64)
    q = qg[:, :, 0, :]
    gate = qg[:, :, 1, :].copy()
    q_out = rope_partial(rmsnorm(q, w_q, eps), positions, rotary_dim, base)
    k_out = rope_partial(rmsnorm(k, w_k, eps), positions, rotary_dim, base)
    return q_out, gate, k_out, np.array(v, np.float64, copy=True)


def output_gate(o, gate):
    """o * sigmoid(gate), elementwise; o and gate [..., D]."""
    o = np.asarray(o, np.float64)
    gate = np.asarray(gate, np.float64)
    return o / (1.0 + np.exp(-gate))
