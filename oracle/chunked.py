"""The same result in 64-token chunks, stage by stage, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page "spark_model/layers/ops/ssm_gdn_a3.rs" (doc comment of
``gdn_prefill_fla``) lists three stages:

1. recompute_wu: the chunk-local cumulative log-gate ``gc``; the strictly
   lower matrix ``L``, which shares its buffer with the key Gram matrix, the
   two in opposite triangles (comment above ``smem_wu``); the
   solves ``(I+L) U = beta V`` and ``(I+L) W = beta exp(gc) K``.  The same
   solves written as one matrix, the UT transform ``T' = (I+L)^-1 diag(beta)``
   (``U = T' V``, ``W = T' diag(exp(gc)) K``), is ``ut_transform``.
2. chunk_delta_h: a serial pass over chunks that emits each chunk's entry
   state and its corrected values ``uc``, and updates the state in place.
3. chunk_fwd_o: ``O = Q~ S_c + tril(decay * Q~ K^T) uc`` per chunk.

The pages give these only as one-line summaries.  The readings taken where
they are open (each one listed with its reason in the design notes):

* ``gc`` is the inclusive prefix sum of ``g`` inside the chunk, restarting at
  every chunk (a global sum would underflow ``exp`` on long sequences).
* ``L[r, s] = beta_r * exp(G_r - G_s) * (k_r . k_s)`` for ``s < r``, else 0.
* ``uc = U - W h_c`` with ``h_c`` the chunk's entry state (stored ``[dk][dv]``).
* The state leaves the chunk as
  ``h_{c+1} = exp(G_n) h_c + K^T diag(exp(G_n - G)) uc`` with ``G_n`` the
  log-gate at the chunk's last token.
* In the output, ``Q~ = diag(exp(G)) Q`` multiplies the entry state, and the
  intra-chunk term uses ``D[r, s] = exp(G_r - G_s)`` on ``Q K^T`` for
  ``s <= r`` (diagonal included: ``o_t`` reads the state after token t).
* No query scale.

Every exponent is taken of a difference ``G_r - G_s`` with ``s <= r``, never of
``-G_s`` alone.  The triangular solves call ``scipy.linalg.solve_triangular``;
the products are numpy matmuls; nothing is blocked, fused or reordered.
"""

import numpy as np
from scipy.linalg import solve_triangular

from .recurrence import kv_head_map


def chunk_cumsum(g_c):
    """Stage 1, gc: inclusive prefix sum of the log-gate over the chunk's
    tokens.  ``g_c`` [n, nv] -> G [n, nv]."""
    return np.cumsum(np.asarray(g_c, dtype=np.float64), axis=0)


def _decay_lower(G, include_diagonal):
    """``D[h, r, s] = exp(G[r, h] - G[s, h])`` on and below (or strictly
    below) the diagonal, 0 elsewhere.  G [n, nv] -> [nv, n, n]."""
    n = G.shape[0]
    r = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    mask = (s <= r) if include_diagonal else (s < r)
    diff = G.T[:, :, None] - G.T[:, None, :]
    return np.where(mask[None], np.exp(np.where(mask[None], diff, 0.0)), 0.0)


def gram_strict_lower(k_c, beta_c, G):
    """Stage 1, L: the key Gram matrix ``A = K K^T`` with its strictly lower
    triangle weighted by ``beta_r exp(G_r - G_s)``.
    ``k_c`` [n, nv, dk] (keys already mapped to v-heads), ``beta_c`` [n, nv]
    -> L [nv, n, n]."""
    k_c = np.asarray(k_c, dtype=np.float64)
    A = np.einsum("rhd,shd->hrs", k_c, k_c)
    beta_c = np.asarray(beta_c, dtype=np.float64)
    return beta_c.T[:, :, None] * _decay_lower(G, include_diagonal=False) * A


def wy_solve(L, k_c, v_c, beta_c, G):
    """Stage 1, the WY/UT solve: ``(I+L) W = diag(beta exp(G)) K`` and
    ``(I+L) U = diag(beta) V``.  Returns W [nv, n, dk], U [nv, n, dv]."""
    k_c = np.asarray(k_c, dtype=np.float64)
    v_c = np.asarray(v_c, dtype=np.float64)
    beta_c = np.asarray(beta_c, dtype=np.float64)
    nv = L.shape[0]
    n = L.shape[1]
    W = np.empty((nv, n, k_c.shape[2]))
    U = np.empty((nv, n, v_c.shape[2]))
    for h in range(nv):
        M = np.eye(n) + L[h]
        rhs_w = (beta_c[:, h] * np.exp(G[:, h]))[:, None] * k_c[:, h, :]
        rhs_u = beta_c[:, h][:, None] * v_c[:, h, :]
        W[h] = solve_triangular(M, rhs_w, lower=True, unit_diagonal=True)
        U[h] = solve_triangular(M, rhs_u, lower=True, unit_diagonal=True)
    return W, U


def ut_transform(L, beta_c):
    """Stage 1, the UT transform: ``T' = (I+L)^-1 diag(beta)``, the matrix that
    maps the right-hand sides of the WY/UT solves to their solutions:
    ``U = T' V`` and ``W = T' diag(exp(G)) K``.  L [nv, n, n], beta_c [n, nv]
    -> T' [nv, n, n] (lower triangular)."""
    beta_c = np.asarray(beta_c, dtype=np.float64)
    nv, n = L.shape[0], L.shape[1]
    out = np.empty((nv, n, n))
    for h in range(nv):
        out[h] = solve_triangular(np.eye(n) + L[h], np.diag(beta_c[:, h]), lower=True, unit_diagonal=True)
    return out


def spine_step(h, W, U, k_c, G):
    """Stage 2, one chunk of the serial spine.  ``h`` [nv, dk, dv] is the
    chunk's entry state.  Returns (uc [nv, n, dv], h_next [nv, dk, dv]) with
    ``uc = U - W h`` and ``h_next = exp(G_n) h + K^T diag(exp(G_n - G)) uc``."""
    k_c = np.asarray(k_c, dtype=np.float64)
    uc = U - np.matmul(W, h)
    Gn = G[-1]                                        # [nv]
    scale = np.exp(Gn[None, :] - G)                   # [n, nv], exponent <= 0
    kw = np.transpose(k_c, (1, 2, 0)) * scale.T[:, None, :]   # [nv, dk, n]
    h_next = np.exp(Gn)[:, None, None] * h + np.matmul(kw, uc)
    return uc, h_next


def chunk_output(q_c, k_c, G, h, uc):
    """Stage 3: ``O = diag(exp(G)) Q h + tril_incl(D * Q K^T) uc`` with
    ``D[r, s] = exp(G_r - G_s)``.  ``q_c``, ``k_c`` [n, nv, dk] -> O [n, nv, dv]."""
    q_c = np.asarray(q_c, dtype=np.float64)
    k_c = np.asarray(k_c, dtype=np.float64)
    Qh = np.transpose(q_c, (1, 0, 2))                 # [nv, n, dk]
    Kh = np.transpose(k_c, (1, 0, 2))
    inter = np.exp(G.T)[:, :, None] * np.matmul(Qh, h)
    P = _decay_lower(G, include_diagonal=True) * np.matmul(Qh, np.transpose(Kh, (0, 2, 1)))
    O = inter + np.matmul(P, uc)
    return np.transpose(O, (1, 0, 2))


def gdn_chunked(q, k, v, g, beta, h0, chunk=64, keep_intermediates=False):
    """One sequence through the three stages.  Arguments as
    ``recurrence.gdn_recurrence``.  Returns (o, h_final, entry, inter) where
    ``inter`` is None or, with ``keep_intermediates``, a list over chunks of
    dicts with ``gc`` [n, nv], ``W`` [nv, n, dk], ``U`` [nv, n, dv],
    ``Tp`` (the UT transform T') [nv, n, n] and ``uc`` [nv, n, dv]
    (n = tokens in that chunk)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, nk, dk = k.shape
    nv, dv = v.shape[1], v.shape[2]
    kappa = kv_head_map(nk, nv)
    h = np.array(h0, dtype=np.float64)
    n_chunks = -(-T // chunk)
    o = np.empty((T, nv, dv))
    entry = np.empty((n_chunks, nv, dk, dv))
    inter = [] if keep_intermediates else None
    for c in range(n_chunks):
        sl = slice(c * chunk, min(T, (c + 1) * chunk))
        q_c, k_c, v_c = q[sl][:, kappa], k[sl][:, kappa], v[sl]
        G = chunk_cumsum(g[sl])
        L = gram_strict_lower(k_c, beta[sl], G)
        W, U = wy_solve(L, k_c, v_c, beta[sl], G)
        entry[c] = h
        uc, h_next = spine_step(h, W, U, k_c, G)
        o[sl] = chunk_output(q_c, k_c, G, h, uc)
        if inter is not None:
            inter.append({"gc": G, "W": W, "U": U, "Tp": ut_transform(L, beta[sl]), "uc": uc})
        h = h_next
    return o, h, entry, inter
