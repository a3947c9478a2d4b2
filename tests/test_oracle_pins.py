"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something the mathematics fixes: a
hand-worked example, closed forms of special cases, a brute-force evaluation
of the recurrence's explicit solution on tiny inputs, and invariants (split,
GQA duplication).  The last group plants plausible mistakes in copies of the
oracle and shows that some pin here rejects each one.
"""

import json
import os

import numpy as np
import pytest

from oracle import gdn_chunked, gdn_recurrence, kv_head_map
from oracle import chunked as chunked_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(rng, T, nk, nv, dk, dv, h0_scale=0.1, unit=True):
    q = rng.standard_normal((T, nk, dk))
    k = rng.standard_normal((T, nk, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, nv, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, nv)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, nv))))
    h0 = h0_scale * rng.standard_normal((nv, dk, dv))
    return q, k, v, g, beta, h0


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------------------
# hand-worked example


def test_hand_worked_three_tokens():
    with open(os.path.join(GOLDEN, "hand_worked_T3.json")) as f:
        gold = json.load(f)
    q = np.array(gold["q"], float)[:, None, :]
    k = np.array(gold["k"], float)[:, None, :]
    v = np.array(gold["v"], float)[:, None, :]
    g = np.log(np.array(gold["g_exp"], float))[:, None]
    beta = np.array(gold["beta"], float)[:, None]
    h0 = np.zeros((1, 2, 2))
    for fn in (gdn_recurrence, lambda *a, **kw: gdn_chunked(*a, **kw)[:3]):
        for C in (1, 2, 64):
            o, hf, _ = fn(q, k, v, g, beta, h0, chunk=C)
            np.testing.assert_allclose(o[:, 0], np.array(gold["o"]), rtol=0, atol=1e-15)
            # stored state is S^T
            np.testing.assert_allclose(hf[0].T, np.array(gold["S_final"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# brute force: the explicit solution of the linear recurrence


def explicit_solution(q, k, v, g, beta, h0):
    """S_t = S_0 A_1...A_t + sum_{s<=t} beta_s v_s k_s^T A_{s+1}...A_t with
    A_u = exp(g_u) (I - beta_u k_u k_u^T); single head, tiny sizes."""
    T, dk = k.shape
    A = [np.exp(g[u]) * (np.eye(dk) - beta[u] * np.outer(k[u], k[u])) for u in range(T)]
    S0 = h0.T
    outs = []
    for t in range(T):
        St = S0.copy()
        for u in range(t + 1):
            St = St @ A[u]
        for s in range(t + 1):
            term = beta[s] * np.outer(v[s], k[s])
            for u in range(s + 1, t + 1):
                term = term @ A[u]
            St = St + term
        outs.append(St @ q[t])
    return np.array(outs), St.T


@pytest.mark.parametrize("dk,dv,T", [(6, 5, 11), (8, 8, 16), (3, 7, 9)])
def test_explicit_solution_bruteforce(dk, dv, T):
    rng = np.random.default_rng(dk * 100 + T)
    q, k, v, g, beta, h0 = rand_problem(rng, T, 1, 1, dk, dv, h0_scale=0.5, unit=False)
    o_ref, h_ref = explicit_solution(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], h0[0])
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0)
    assert rel(o[:, 0], o_ref) < 1e-12
    assert rel(hf[0], h_ref) < 1e-12
    for C in (1, 4, 5, T):
        o2, hf2, _, _ = gdn_chunked(q, k, v, g, beta, h0, chunk=C)
        assert rel(o2[:, 0], o_ref) < 1e-12
        assert rel(hf2[0], h_ref) < 1e-12


# ---------------------------------------------------------------------------
# two algorithms: token recurrence vs WY/UT chunk form


@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunked_equals_recurrence(C):
    rng = np.random.default_rng(7)
    q, k, v, g, beta, h0 = rand_problem(rng, 150, 2, 4, 16, 12)
    o, hf, ent = gdn_recurrence(q, k, v, g, beta, h0, chunk=C)
    o2, hf2, ent2, _ = gdn_chunked(q, k, v, g, beta, h0, chunk=C)
    assert rel(o2, o) < 1e-12 and rel(hf2, hf) < 1e-12 and rel(ent2, ent) < 1e-12


def test_chunked_equals_recurrence_head_dim_128():
    rng = np.random.default_rng(8)
    q, k, v, g, beta, h0 = rand_problem(rng, 200, 1, 2, 128, 128, h0_scale=0.02)
    o, hf, ent = gdn_recurrence(q, k, v, g, beta, h0)
    o2, hf2, ent2, _ = gdn_chunked(q, k, v, g, beta, h0)
    assert rel(o2, o) < 1e-12 and rel(hf2, hf) < 1e-12 and rel(ent2, ent) < 1e-12


# ---------------------------------------------------------------------------
# closed forms of special cases


def test_beta_zero_is_pure_decay():
    """beta = 0: nothing is written, S_t = exp(sum g) S_0 and
    o_t = exp(G_t) S_0 q_t with G the running sum of g."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, h0 = rand_problem(rng, 90, 2, 2, 8, 8)
    beta[:] = 0
    G = np.cumsum(g, axis=0)
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0)
    kap = kv_head_map(2, 2)
    expect = np.exp(G)[:, :, None] * np.einsum("hkd,thk->thd", h0, q[:, kap])
    assert rel(o, expect) < 1e-13
    assert rel(hf, np.exp(G[-1])[:, None, None] * h0) < 1e-13
    o2, hf2, _, _ = gdn_chunked(q, k, v, g, beta, h0, chunk=16)
    assert rel(o2, expect) < 1e-13


def test_one_hot_keys_overwrite():
    """g = 0, beta = 1, k_t = e_{pi(t)}: each token replaces column pi(t) of S
    (row pi(t) of the stored h) with v_t; untouched rows keep h0."""
    rng = np.random.default_rng(2)
    dk, dv, T = 8, 5, 20
    pi = rng.integers(0, dk - 2, size=T)          # rows dk-2, dk-1 never written
    k = np.eye(dk)[pi][:, None, :]
    q = np.eye(dk)[rng.integers(0, dk, size=T)][:, None, :]
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    h0 = rng.standard_normal((1, dk, dv))
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0)
    h = h0[0].copy()
    for t in range(T):
        h[pi[t]] = v[t, 0]
        np.testing.assert_allclose(o[t, 0], h[np.argmax(q[t, 0])], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hf[0], h, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(hf[0][dk - 2:], h0[0][dk - 2:])


@pytest.mark.parametrize("key_kind", ["one_hot", "pm_0.125_x64", "pm_0.5_x4"])
def test_q_equals_k_beta_one_returns_v(key_kind):
    """beta = 1, q = k with |k| = 1 exactly: S_t k_t = v_t for any g and S_0."""
    rng = np.random.default_rng(3)
    dk, T, nv = 128, 100, 2
    k = np.zeros((T, 1, dk))
    for t in range(T):
        if key_kind == "one_hot":
            k[t, 0, rng.integers(dk)] = 1.0
        elif key_kind == "pm_0.125_x64":
            idx = rng.choice(dk, 64, replace=False)
            k[t, 0, idx] = 0.125 * rng.choice([-1.0, 1.0], 64)
        else:
            idx = rng.choice(dk, 4, replace=False)
            k[t, 0, idx] = 0.5 * rng.choice([-1.0, 1.0], 4)
    v = rng.standard_normal((T, nv, 128))
    g = -np.logaddexp(0, rng.standard_normal((T, nv)))
    beta = np.ones((T, nv))
    h0 = rng.standard_normal((nv, dk, 128))
    o, _, _ = gdn_recurrence(k, k, v, g, beta, h0)
    assert np.abs(o - v).max() < 1e-12
    o2, _, _, _ = gdn_chunked(k, k, v, g, beta, h0)
    assert np.abs(o2 - v).max() < 1e-10


def test_orthogonal_keys_reduce_to_gated_linear_attention():
    """h0 = 0 and mutually orthogonal keys: the erase term never touches
    another token's write, so O = tril_incl(D * Q K^T) diag(beta) V with
    D[r, s] = exp(G_r - G_s) -- masked, gated linear attention in O(T^2)."""
    rng = np.random.default_rng(4)
    dk, dv, T = 32, 16, 24
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = (basis[:T] * rng.uniform(0.5, 1.5, size=(T, 1)))[:, None, :]
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = -np.logaddexp(0, rng.standard_normal((T, 1)))
    beta = rng.uniform(0.1, 1.0, size=(T, 1))
    G = np.cumsum(g[:, 0])
    D = np.tril(np.exp(G[:, None] - G[None, :]))
    expect = (D * (q[:, 0] @ k[:, 0].T)) @ (beta[:, 0][:, None] * v[:, 0])
    o, _, _ = gdn_recurrence(q, k, v, g, beta, np.zeros((1, dk, dv)))
    assert rel(o[:, 0], expect) < 1e-12


def test_strong_forgetting():
    """g = -80: the carried state is scaled by e^-80 each token, so
    o_t = beta_t (k_t . q_t) v_t and the final stored state is
    beta_T k_T v_T^T, up to e^-80 relative (below float64 rounding)."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, h0 = rand_problem(rng, 40, 1, 1, 16, 16, h0_scale=1.0)
    g[:] = -80.0
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0)
    expect = beta[:, 0, None] * np.sum(k[:, 0] * q[:, 0], axis=1)[:, None] * v[:, 0]
    assert rel(o[:, 0], expect) < 1e-14   # e^-80 is far below rounding
    assert rel(hf[0], beta[-1, 0] * np.outer(k[-1, 0], v[-1, 0])) < 1e-14


def test_empty_sequence_keeps_state():
    q = np.zeros((0, 1, 8))
    v = np.zeros((0, 2, 8))
    g = np.zeros((0, 2))
    h0 = np.random.default_rng(0).standard_normal((2, 8, 8))
    o, hf, ent = gdn_recurrence(q, q, v, g, g, h0)
    assert o.shape == (0, 2, 8) and ent.shape[0] == 0
    np.testing.assert_array_equal(hf, h0)
    o2, hf2, ent2, _ = gdn_chunked(q, q, v, g, g, h0)
    np.testing.assert_array_equal(hf2, h0)


# ---------------------------------------------------------------------------
# invariants


@pytest.mark.parametrize("T1", [64, 100, 1])
def test_split_invariance_and_entry_states(T1):
    """Running [0, T) equals running [0, T1) and then [T1, T) from the carried
    state; entry state c equals the final state of the first 64c tokens."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, h0 = rand_problem(rng, 200, 2, 4, 12, 10)
    o, hf, ent = gdn_recurrence(q, k, v, g, beta, h0)
    oa, ha, _ = gdn_recurrence(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], h0)
    ob, hb, _ = gdn_recurrence(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], ha)
    assert rel(np.concatenate([oa, ob]), o) < 1e-12 and rel(hb, hf) < 1e-12
    for c in range(ent.shape[0]):
        _, hc, _ = gdn_recurrence(q[:64 * c], k[:64 * c], v[:64 * c], g[:64 * c], beta[:64 * c], h0)
        assert rel(ent[c], hc) < 1e-12


def test_gqa_equals_duplicated_k_heads():
    """nk < nv gives the same result as nk = nv with each k-head copied to
    the v-heads that read it (kappa(h) = h*nk//nv)."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, h0 = rand_problem(rng, 70, 2, 6, 8, 8)
    kap = kv_head_map(2, 6)
    assert list(kap) == [0, 0, 0, 1, 1, 1]
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0)
    o2, hf2, _ = gdn_recurrence(q[:, kap], k[:, kap], v, g, beta, h0)
    assert rel(o, o2) < 1e-15 and rel(hf, hf2) < 1e-15


# ---------------------------------------------------------------------------
# planted mistakes: each mutant must be rejected by a pin above


def mutant_recurrence(q, k, v, g, beta, h0, mistake):
    T, nk, dk = k.shape
    kap = kv_head_map(nk, v.shape[1])
    # the stored state is h = S^T; the mutant "transposed_state" forgets that
    S = h0.copy() if mistake == "transposed_state" else np.swapaxes(h0, 1, 2).copy()
    o = np.empty(v.shape)
    for t in range(T):
        kt, qt = k[t, kap], q[t, kap]
        a = np.exp(g[t])[:, None, None] if mistake != "no_decay" else 1.0
        b = beta[t][:, None, None]
        sign = -1.0 if mistake != "erase_sign" else 1.0
        Sk = np.matmul(S, kt[:, :, None])
        S_new = a * (S + sign * b * Sk * kt[:, None, :]) + b * v[t][:, :, None] * kt[:, None, :]
        src = S if mistake == "output_before_update" else S_new
        o[t] = np.matmul(src, qt[:, :, None])[:, :, 0]
        S = S_new
    hf = S if mistake == "transposed_state" else np.swapaxes(S, 1, 2)
    return o, hf


@pytest.mark.parametrize("mistake", ["no_decay", "erase_sign", "output_before_update", "transposed_state"])
def test_pins_reject_planted_recurrence_mistakes(mistake):
    rng = np.random.default_rng(11)
    rejected = []
    # q = k, beta = 1 -> o = v
    dk = 8
    k = np.eye(dk)[rng.integers(dk, size=30)][:, None, :]
    v = rng.standard_normal((30, 1, dk))
    g = -np.logaddexp(0, rng.standard_normal((30, 1)))
    h0 = rng.standard_normal((1, dk, dk))
    o, _ = mutant_recurrence(k, k, v, g, np.ones((30, 1)), h0, mistake)
    rejected.append(np.abs(o - v).max() > 1e-6)
    # beta = 0 closed form
    q2, k2, v2, g2, b2, h02 = rand_problem(rng, 30, 1, 1, dk, dk)
    b2[:] = 0
    o2, _ = mutant_recurrence(q2, k2, v2, g2, b2, h02, mistake)
    G = np.cumsum(g2, axis=0)
    expect = np.exp(G)[:, :, None] * np.einsum("hkd,thk->thd", h02, q2)
    rejected.append(rel(o2, expect) > 1e-6)
    # hand-worked example
    with open(os.path.join(GOLDEN, "hand_worked_T3.json")) as f:
        gold = json.load(f)
    o3, h3 = mutant_recurrence(np.array(gold["q"], float)[:, None], np.array(gold["k"], float)[:, None],
                               np.array(gold["v"], float)[:, None],
                               np.log(np.array(gold["g_exp"], float))[:, None],
                               np.array(gold["beta"], float)[:, None], np.zeros((1, 2, 2)), mistake)
    rejected.append(np.abs(o3[:, 0] - np.array(gold["o"])).max() > 1e-9
                    or np.abs(h3[0].T - np.array(gold["S_final"])).max() > 1e-9)
    assert any(rejected), f"no pin rejects the planted mistake {mistake!r}"


@pytest.mark.parametrize("mistake", ["strict_output_mask", "decay_from_first_token", "no_entry_decay_in_output"])
def test_pins_reject_planted_chunk_form_mistakes(mistake, monkeypatch):
    """Plant a mistake in the chunk form's stages; chunked == recurrence fails."""
    if mistake == "strict_output_mask":
        orig = chunked_mod._decay_lower
        monkeypatch.setattr(chunked_mod, "_decay_lower", lambda G, include_diagonal: orig(G, False))
    elif mistake == "decay_from_first_token":
        orig_step = chunked_mod.spine_step
        monkeypatch.setattr(chunked_mod, "spine_step",
                            lambda h, W, U, k_c, G: orig_step(h, W, U, k_c, G[::-1]))
    else:
        monkeypatch.setattr(chunked_mod, "chunk_output", _output_without_entry_decay)
    rng = np.random.default_rng(12)
    q, k, v, g, beta, h0 = rand_problem(rng, 100, 1, 2, 16, 16, h0_scale=0.5)
    o, hf, _ = gdn_recurrence(q, k, v, g, beta, h0, chunk=32)
    o2, hf2, _, _ = chunked_mod.gdn_chunked(q, k, v, g, beta, h0, chunk=32)
    assert rel(o2, o) > 1e-6 or rel(hf2, hf) > 1e-6


def _output_without_entry_decay(q_c, k_c, G, h, uc):
    Qh = np.transpose(q_c, (1, 0, 2))
    Kh = np.transpose(k_c, (1, 0, 2))
    P = chunked_mod._decay_lower(G, True) * np.matmul(Qh, np.transpose(Kh, (0, 2, 1)))
    return np.transpose(np.matmul(Qh, h) + np.matmul(P, uc), (1, 0, 2))


def test_ut_transform_reproduces_the_direct_solves():
    """T' = (I+L)^-1 diag(beta) maps the right-hand sides to the solutions of
    the direct triangular solves: U = T' V and W = T' diag(exp(G)) K; and
    (I+L) T' = diag(beta) holds to rounding."""
    rng = np.random.default_rng(31)
    q, k, v, g, beta, h0 = rand_problem(rng, 64, 1, 3, 128, 128)
    kap = kv_head_map(1, 3)
    k_c = k[:, kap]
    G = chunked_mod.chunk_cumsum(g)
    L = chunked_mod.gram_strict_lower(k_c, beta, G)
    W, U = chunked_mod.wy_solve(L, k_c, v, beta, G)
    Tp = chunked_mod.ut_transform(L, beta)
    for h in range(3):
        assert rel(Tp[h] @ v[:, h], U[h]) < 1e-12
        assert rel(Tp[h] @ (np.exp(G[:, h])[:, None] * k_c[:, h]), W[h]) < 1e-12
        assert rel((np.eye(64) + L[h]) @ Tp[h], np.diag(beta[:, h])) < 1e-12
        assert np.all(np.triu(Tp[h], 1) == 0)


def test_ut_transform_is_the_neumann_series():
    """L is strictly lower triangular, hence nilpotent (L^n = 0 for n rows), so
    (I+L)^-1 is exactly the finite Neumann sum I - L + L^2 - ... + (-L)^(n-1):
    T' = (sum_j (-L)^j) diag(beta), formed by matrix powers, a different
    algorithm from the inverse; and for two tokens, by hand,
    T' = [[b0, 0], [-L10 b0, b1]]."""
    rng = np.random.default_rng(41)
    q, k, v, g, beta, h0 = rand_problem(rng, 64, 1, 2, 128, 128)
    k_c = k[:, kv_head_map(1, 2)]
    G = chunked_mod.chunk_cumsum(g)
    L = chunked_mod.gram_strict_lower(k_c, beta, G)
    Tp = chunked_mod.ut_transform(L, beta)
    for h in range(2):
        term = np.eye(64)
        series = np.eye(64)
        for _ in range(63):
            term = -term @ L[h]
            series = series + term
        assert np.all(term @ L[h] == 0)  # L^64 = 0
        assert rel(Tp[h], series * beta[:, h][None, :]) < 1e-12
    L2 = np.array([[[0.0, 0.0], [0.375, 0.0]]])
    b2 = np.array([[0.5], [0.25]])
    assert np.array_equal(chunked_mod.ut_transform(L2, b2)[0], np.array([[0.5, 0.0], [-0.1875, 0.25]]))
