"""The definition: the gated delta rule, token by token, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg, never by the
product path.

The gated delta rule (Gated DeltaNet), per value head:

    S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

with S in R^{dv x dk}.  This is the method the page
"spark_model/layers/ops/ssm_gdn_a3.rs" runs as its GDN prefill (its kernels
are the gated_delta_rule_chunk_* family, its stages listed in the doc comment
of ``gdn_prefill_fla``); the page stores the state as ``[kd][vd]``
(comment on ``h_state_is_table``), i.e. ``h = S^T``; inputs and outputs of this
module use that stored orientation, the loop itself uses S.

``S (I - beta k k^T)`` is evaluated as ``S - beta (S k) k^T``: the same product
with the rank-one factor applied by associativity, no other reordering.
"""

import numpy as np


def kv_head_map(nk, nv):
    """k-head read by each v-head.  The pages give separate ``num_k_heads`` and
    ``num_v_heads`` (``gdn_prefill_fla`` arguments) but not the mapping; the
    reading taken here is that consecutive v-heads share a k-head:
    ``kappa(h) = (h * nk) // nv`` with ``nv % nk == 0``.  Parity unpinned: a
    convention, shared with the GPU library through documentation only."""
    if nk <= 0 or nv % nk != 0:
        raise ValueError("nv must be a positive multiple of nk")
    return (np.arange(nv) * nk) // nv


def gdn_recurrence(q, k, v, g, beta, h0, chunk=64):
    """Run one sequence through the recurrence.

    Arguments (any float dtype; converted exactly to float64):
      q, k  : [T, nk, dk]   queries and keys per k-head
      v     : [T, nv, dv]   values per v-head
      g     : [T, nv]       log-gate (exp(g) is the decay)
      beta  : [T, nv]       write strength
      h0    : [nv, dk, dv]  initial state in stored orientation (h = S^T)
      chunk : boundary spacing at which entry states are recorded

    Returns (o [T, nv, dv], h_final [nv, dk, dv], entry [ceil(T/chunk), nv, dk, dv]).
    ``entry[c]`` is the state before token ``c*chunk`` (so ``entry[0] = h0``):
    the per-chunk entry states the page's spine emits (doc comment of
    ``gdn_prefill_fla``, stage 2).  A length-0 sequence returns ``h_final = h0``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, nk, dk = k.shape
    nv, dv = v.shape[1], v.shape[2]
    kappa = kv_head_map(nk, nv)

    S = np.ascontiguousarray(np.swapaxes(np.asarray(h0, dtype=np.float64), 1, 2))  # [nv, dv, dk]
    n_chunks = -(-T // chunk)
    o = np.empty((T, nv, dv))
    entry = np.empty((n_chunks, nv, dk, dv))
    for t in range(T):
        if t % chunk == 0:
            entry[t // chunk] = np.swapaxes(S, 1, 2)
        kt = k[t, kappa]                      # [nv, dk]
        qt = q[t, kappa]                      # [nv, dk]
        a = np.exp(g[t])[:, None, None]       # decay
        b = beta[t][:, None, None]
        Sk = np.matmul(S, kt[:, :, None])     # [nv, dv, 1] = S k
        S = a * (S - b * Sk * kt[:, None, :]) + b * v[t][:, :, None] * kt[:, None, :]
        o[t] = np.matmul(S, qt[:, :, None])[:, :, 0]   # o_t = S_t q_t
    return o, np.ascontiguousarray(np.swapaxes(S, 1, 2)), entry
