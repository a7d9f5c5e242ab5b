"""Gated delta rule state update (fp64 definition) and its chunkwise form.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source passages
---------------
* 24-ai.news TokenSpeed article, paragraph on the model: the linear-attention
  layers of the hybrid model are Gated DeltaNet (GDN) layers.
* zubnet.ai TokenSpeed article, second paragraph: those layers keep a
  recurrent state that is checkpointed next to the KV in state slots and
  reached through an index array (``current_input_indices``) instead of
  tensor copies.
* 24-ai.news, optimisation list, "Mamba State Update": the intermediate state
  copy is removed by index indirection, an O(1) pointer update.

The recurrence is the published gated delta rule (Yang, Kautz & Hatamizadeh,
"Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025):

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

with S in R^{d_v x d_k}.  ``step`` evaluates exactly that formula with the
dense (I - beta k k^T) matrix.

Readings (pages silent): the output is o = q_scale * S q with S in
d_v x d_k (the retrieval property S_t k_t = v_t for beta = 1, |k| = 1 fixes
the orientation); q_scale = 1 by default; alpha and beta arrive as per
(token, head) values; q and k arrive L2-normalised; heads are independent;
slot index -1 means a zero initial state.  State pools are float32
[n_slots, H, d_v, d_k]; a checkpoint is the float32 rounding (nearest even)
of the float64 state.
"""

import numpy as np


def gates_from_raw(g, b):
    """Per-(token, head) gates from their raw values: alpha = exp(g) (g is the
    log decay, g <= 0) and beta = 1 / (1 + exp(-b)), the parameterisation of
    the Gated DeltaNet paper (decay in (0, 1], write strength in (0, 1)).
    Reading (pages silent): the kernel receives g and b as they leave the
    layer's projections."""
    g = np.asarray(g, np.float64)
    b = np.asarray(b, np.float64)
    # the logistic function in its two-branch form (exp of -|b| only, so no
    # overflow for large |b|): 1 / (1 + e^-b) for b >= 0, e^b / (1 + e^b) below
    e = np.exp(-np.abs(b))
    return np.exp(g), np.where(b >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def step(S, q, k, v, alpha, beta):
    """One token of the recurrence, dense form.  Returns (S_t, S_t q)."""
    d_k = k.shape[0]
    A = np.eye(d_k) - beta * np.outer(k, k)
    S_new = alpha * (S @ A) + beta * np.outer(v, k)
    return S_new, S_new @ q


def sequential(S0, q, k, v, alpha, beta, q_scale=1.0):
    """Run T tokens from S0.  q, k [T, d_k]; v [T, d_v]; alpha, beta [T].

    Returns (states [T, d_v, d_k], outputs [T, d_v]).
    """
    S = np.asarray(S0, np.float64)
    T = q.shape[0]
    states = np.empty((T,) + S.shape)
    outs = np.empty((T, S.shape[0]))
    for t in range(T):
        S, o = step(S, np.asarray(q[t], np.float64), np.asarray(k[t], np.float64),
                    np.asarray(v[t], np.float64), float(alpha[t]), float(beta[t]))
        states[t] = S
        outs[t] = q_scale * o
    return states, outs


def sequential_heads(S0, q, k, v, alpha, beta, q_scale=1.0):
    """All heads of one sequence over T tokens, in the rank-one form.

    S (I - beta k k^T) = S - beta (S k) k^T, so each token costs O(d_v d_k)
    per head instead of the dense product's O(d_v d_k^2); the result is the
    same recurrence as ``step`` (pinned against it to 1e-12).  S0 [H, d_v,
    d_k]; q, k [T, H, d_k]; v [T, H, d_v]; alpha, beta [T, H].  Returns
    (final state [H, d_v, d_k], outputs [T, H, d_v]); intermediate states are
    not kept, so a long chain stays cheap in memory.
    """
    S = np.array(S0, np.float64, copy=True)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    outs = np.empty((T,) + v.shape[1:])
    for t in range(T):
        Sk = np.einsum("hvk,hk->hv", S, k[t])
        S = alpha[t][:, None, None] * (S - beta[t][:, None, None] * Sk[:, :, None] * k[t][:, None, :]) \
            + beta[t][:, None, None] * v[t][:, :, None] * k[t][:, None, :]
        outs[t] = q_scale * np.einsum("hvk,hk->hv", S, q[t])
    return S, outs


def chunked(S0, q, k, v, alpha, beta, chunk, q_scale=1.0):
    """The same recurrence evaluated chunk by chunk (WY / UT form).

    Within a chunk of C tokens starting from S0, with gamma_t = prod_{i<=t}
    alpha_i, the delta-rule inputs u_t (S_t = alpha_t S_{t-1} + u_t k_t^T)
    solve the unit lower-triangular system
        u_t + beta_t sum_{i<t} (gamma_t/gamma_i)(k_t . k_i) u_i
            = beta_t (v_t - gamma_t S0 k_t),
    and then  S_C = gamma_C S0 + sum_i (gamma_C/gamma_i) u_i k_i^T,
              o_t = gamma_t S0 q_t + sum_{i<=t} (gamma_t/gamma_i)(k_i . q_t) u_i.
    (Yang et al., "Parallelizing Linear Transformers with the Delta Rule
    over Sequence Length", NeurIPS 2024, and the Gated DeltaNet paper above;
    derived here from the recurrence.)  Ratios use log-space cumulative sums.
    Returns (final state, outputs [T, d_v]).
    """
    S = np.asarray(S0, np.float64)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    outs = np.empty((T, S.shape[0]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        K, Q, Vv = k[c0:c1], q[c0:c1], v[c0:c1]
        b = beta[c0:c1]
        lg = np.cumsum(np.log(alpha[c0:c1]))                  # log gamma_t
        C = c1 - c0
        ratio = np.exp(lg[:, None] - lg[None, :])             # gamma_t / gamma_i
        KK = K @ K.T
        rhs = b[:, None] * (Vv - np.exp(lg)[:, None] * (K @ S.T))
        U = np.zeros_like(rhs)
        for t in range(C):                                     # forward substitution
            acc = rhs[t].copy()
            for i in range(t):
                acc -= b[t] * ratio[t, i] * KK[t, i] * U[i]
            U[t] = acc
        KQ = K @ Q.T                                           # [i, t] = k_i . q_t
        for t in range(C):
            o = np.exp(lg[t]) * (S @ Q[t])
            for i in range(t + 1):
                o = o + ratio[t, i] * KQ[i, t] * U[i]
            outs[c0 + t] = q_scale * o
        gC = np.exp(lg[-1])
        S = gC * S + (U * np.exp(lg[-1] - lg)[:, None]).T @ K
    return S, outs


def state_update(pool, in_idx, out_idx, q, k, v, alpha, beta, q_scale=1.0):
    """Slot-addressed batched update, the operation of one GDN layer.

    pool float32 [n_slots, H, d_v, d_k]; in_idx [S]; out_idx [S, T];
    q, k [S, T, H, d_k] and v [S, T, H, d_v] float64; alpha, beta [S, T, H].
    Every input slot is read from ``pool`` as it was before the call; after
    token t the float32 state is written to slot out_idx[s, t].  Returns
    (new pool, o float64 [S, T, H, d_v]).
    """
    pool = np.asarray(pool, np.float32)
    new_pool = pool.copy()
    S_n, T = out_idx.shape
    H, d_v, d_k = pool.shape[1:]
    o = np.empty((S_n, T, H, d_v))
    for s in range(S_n):
        for h in range(H):
            if in_idx[s] < 0:
                S0 = np.zeros((d_v, d_k))
            else:
                S0 = pool[in_idx[s], h].astype(np.float64)
            states, outs = sequential(S0, q[s, :, h], k[s, :, h], v[s, :, h],
                                      alpha[s, :, h], beta[s, :, h], q_scale)
            o[s, :, h] = outs
            for t in range(T):
                new_pool[out_idx[s, t], h] = states[t].astype(np.float32)
    return new_pool, o


def prefill(pool, in_idx, out_idx, cu_seqlens, q, k, v, alpha, beta, q_scale=1.0):
    """Slot-addressed prefill of a batch of variable-length sequences.

    The operation a GDN layer performs on a prompt (the turn inputs and the
    long first turn of the agentic workload): sequence s owns tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed inputs, starts from
    slot in_idx[s] (zero state for -1), runs the recurrence over all of its
    tokens and writes only its final state, as float32, to slot out_idx[s].
    A sequence with no token copies its input state.  Every input slot is
    read as it was before the call.

    pool float32 [n_slots, H, d_v, d_k]; q, k [N, H, d_k]; v [N, H, d_v];
    alpha, beta [N, H] (float64 values).  Returns (new pool, o [N, H, d_v]).
    """
    pool = np.asarray(pool, np.float32)
    new_pool = pool.copy()
    H, d_v, d_k = pool.shape[1:]
    o = np.empty((q.shape[0], H, d_v))
    finals = []
    for s in range(len(in_idx)):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        S0 = np.zeros((H, d_v, d_k)) if in_idx[s] < 0 else pool[in_idx[s]].astype(np.float64)
        S, o[a:b] = sequential_heads(S0, q[a:b], k[a:b], v[a:b], alpha[a:b], beta[a:b], q_scale)
        finals.append(S)
    for s, S in enumerate(finals):
        new_pool[out_idx[s]] = S.astype(np.float32)
    return new_pool, o
