"""Comparison of the GPU library with the oracle (helpers for the gpu tests).

Tolerances (written here once, used by every parity test):
  * outputs o (bf16): max |o_gpu - o_ref| <= 2e-2
  * final state (f32): relative Frobenius error <= 1e-3 per (sequence, head)
  * entry states (bf16): max abs <= 2e-2, relative Frobenius <= 4e-3
    (bf16 storage alone is ~2^-9 relative)
  * gc: |err| <= 1e-4 * (1 + |G|)   (64 float32 additions)
  * T' (stored as a bf16 hi + lo pair, ~2^-17 relative per element, on top of
    the solve's hi/lo products, <= 2^-16): relative Frobenius <= 1e-4 per
    slot; W and U rebuilt from it (U = T' V, W = T' diag(exp(G)) K): <= 1e-4
    against the oracle's direct triangular solves
  * row scales 1/|k_t|, 1/|q_t| (with q/k normalisation): relative <= 1e-5
    (a float32 sum of 128 squares and a reciprocal square root)
"""

import os

import numpy as np

from oracle import gdn_chunked, gdn_recurrence, kv_head_map, l2_normalize
from oracle.chunked import chunk_cumsum, gram_strict_lower, ut_transform, wy_solve
from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64

TOL_O_MAXABS = 2e-2
TOL_STATE_RELFRO = 1e-3
TOL_ENTRY_MAXABS = 2e-2
TOL_ENTRY_RELFRO = 4e-3
TOL_WU_RELFRO = 1e-4
TOL_TP_RELFRO = 1e-4
TOL_NRM_REL = 1e-5
OPT_ENTRY_STATES = 0x1  # include/gdn_prefill.h
OPT_L2NORM_QK = 0x2


def relfro(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# element offset of fragment f, and whether it keeps only the first 4 values
# per lane (the diagonal fragments f = 0, 4, whose other half lies above the
# diagonal)
_TP_OFF = (0, 256, 768, 1280, 1792, 2048)
_TP_HALF = (True, False, False, False, True, False)


def _tp_index():
    """Row / column of each stored element of a slot's T' (2560 values): fragment
    f of the six lower-triangular (mt, kb) (f = mt for kb = 0, f = mt + 2 for
    kb = 1), lane 16q + r holds row 16mt + r, columns 32kb + 4q + e and
    32kb + 16 + 4q + e; the diagonal fragments hold only the first four."""
    t = np.zeros(2560, dtype=np.int64)
    sc = np.zeros(2560, dtype=np.int64)
    for mt in range(4):
        for kb in range(2):
            if 2 * kb > mt:
                continue
            f = mt if kb == 0 else mt + 2
            per = 4 if _TP_HALF[f] else 8
            for lane in range(64):
                q, r = lane // 16, lane % 16
                for e in range(per):
                    i = _TP_OFF[f] + lane * per + e
                    t[i] = 16 * mt + r
                    sc[i] = 32 * kb + (4 * q + e if e < 4 else 16 + 4 * q + e - 4)
    return t, sc


_TP_T, _TP_S = _tp_index()


def unpack_tp(vals):
    """T' [64, 64] from the documented layout [2][2560] (bf16 hi, then lo, as
    float values); elements not stored are 0."""
    vals = np.asarray(vals, dtype=np.float64)
    T = np.zeros((64, 64))
    T[_TP_T, _TP_S] = vals[0] + vals[1]
    return T


def seq_arrays(p, i, heads=None, cu=None, normalize=False):
    """Oracle inputs of sequence i restricted to v-heads ``heads``; the k-heads
    are selected with the documented grouping so the oracle sees nk = nv.
    ``cu``: p.cu_seqlens, when the caller already holds it.  ``normalize``: q
    and k normalised per token by the oracle (for calls with q/k
    normalisation)."""
    cu = p.cu_seqlens if cu is None else cu
    a, b = int(cu[i]), int(cu[i + 1])
    heads = list(range(p.nv)) if heads is None else list(heads)
    kap = kv_head_map(p.nk, p.nv)[heads]
    q, k = bf16_to_f64(p.q[a:b][:, kap]), bf16_to_f64(p.k[a:b][:, kap])
    if normalize:
        q, k = l2_normalize(q), l2_normalize(k)
    return dict(q=q, k=k, v=bf16_to_f64(p.v[a:b][:, heads]), g=p.g[a:b][:, heads].astype(np.float64),
                beta=p.beta[a:b][:, heads].astype(np.float64), h0=p.h0[i][heads].astype(np.float64))


def check_problem(dp, p, seqs=None, heads=None, intermediates=False, entries=None, report=None,
                  chunked=False):
    """Run the oracle on (seqs x heads) and compare with what the GPU left in
    ``dp`` (output, final state, scratch).  The oracle is the token recurrence,
    or its chunk form when ``chunked`` or ``intermediates`` is set (the two
    agree to 1e-12, a CPU pin; the chunk form runs many heads of a long
    sequence several times faster).  ``entries`` (default: whether the call
    emitted them) compares the entry states.  Returns a dict of worst errors."""
    if entries is None:
        entries = bool(getattr(dp, "flags", OPT_ENTRY_STATES) & OPT_ENTRY_STATES)
    seqs = range(p.nseq) if seqs is None else seqs
    heads_l = list(range(p.nv)) if heads is None else list(heads)
    norm = bool(getattr(dp, "flags", 0) & OPT_L2NORM_QK)
    worst = dict(o_maxabs=0.0, state_relfro=0.0, entry_maxabs=0.0, entry_relfro=0.0,
                 w_relfro=0.0, u_relfro=0.0, tp_relfro=0.0, gc_err=0.0, nrm_err=0.0)
    regions = {}
    if entries:
        regions["s_entry"] = dp.region("s_entry")
    if intermediates:
        for r in ("gc", "tp") + (("nrm",) if norm else ()):
            regions[r] = dp.region(r)
    cu = p.cu_seqlens
    for i in seqs:
        a = int(cu[i])
        L = int(p.lengths[i])
        arrs = seq_arrays(p, i, heads_l, cu, normalize=norm)
        raw = seq_arrays(p, i, heads_l, cu) if (norm and intermediates) else arrs
        if intermediates:
            o_ref, h_ref, ent_ref, inter = gdn_chunked(**arrs, keep_intermediates=True)
        elif chunked:
            o_ref, h_ref, ent_ref, _ = gdn_chunked(**arrs)
        else:
            o_ref, h_ref, ent_ref = gdn_recurrence(**arrs)
        if L:
            o_gpu = dp.output_rows(a, a + L, heads_l)
            worst["o_maxabs"] = max(worst["o_maxabs"], float(np.abs(o_gpu - o_ref).max()))
        state_i = dp.state_of(i)
        for j, h in enumerate(heads_l):
            e = relfro(state_i[h].astype(np.float64), h_ref[j])
            worst["state_relfro"] = max(worst["state_relfro"], e)
            for c in range(ent_ref.shape[0]):
                sl = dp.slot(i, h, c)
                if "s_entry" in regions:
                    # stored as S = h^T ([dv][dk])
                    s_gpu = regions["s_entry"][sl].float().cpu().numpy().astype(np.float64).T
                    worst["entry_maxabs"] = max(worst["entry_maxabs"], float(np.abs(s_gpu - ent_ref[c, j]).max()))
                    worst["entry_relfro"] = max(worst["entry_relfro"], relfro(s_gpu, ent_ref[c, j]))
                if intermediates:
                    d = inter[c]
                    rows = slice(64 * c, 64 * c + 64)
                    _compare_slot(regions, sl, d["gc"][:, j], d["Tp"][j], d["W"][j], d["U"][j],
                                  arrs["k"][rows, j], arrs["v"][rows, j], worst,
                                  raw_qk=(raw["q"][rows, j], raw["k"][rows, j]) if norm else None)
    if report is not None:
        report.update(worst)
    return worst


def _compare_slot(regions, sl, G, Tp_ref, W_ref, U_ref, kk, vv, worst, raw_qk=None):
    """Stage-1 intermediates of one slot (n = len(G) tokens) against the
    oracle's: gc, T' (padded rows and columns exactly 0), W, U rebuilt from
    the GPU's T', and with q/k normalisation the row scales 1/|k_t|, 1/|q_t|
    against the raw rows ``raw_qk`` = (q, k)."""
    n = len(G)
    gc_gpu = regions["gc"][sl].cpu().numpy().astype(np.float64)
    worst["gc_err"] = max(worst["gc_err"], float((np.abs(gc_gpu[:n] - G) / (1 + np.abs(G))).max()))
    # rows past the end repeat the last value
    worst["gc_err"] = max(worst["gc_err"], float(np.abs(gc_gpu[n:] - G[-1]).max(initial=0)))
    if raw_qk is not None:
        nrm = regions["nrm"][sl].cpu().numpy().astype(np.float64)
        for part, x in ((0, raw_qk[1]), (1, raw_qk[0])):
            norm = np.linalg.norm(np.asarray(x, np.float64)[:n], axis=-1)
            ref = np.divide(1.0, norm, out=np.zeros_like(norm), where=norm > 0)
            err = np.abs(nrm[part, :n] - ref) / np.maximum(ref, 1e-30)
            worst["nrm_err"] = max(worst["nrm_err"], float(np.where(ref > 0, err, nrm[part, :n] != 0).max()))
            # rows past the end repeat the last row's scale
            worst["nrm_err"] = max(worst["nrm_err"], float(np.abs(nrm[part, n:] - nrm[part, n - 1]).max(initial=0)))
    Tp = unpack_tp(regions["tp"][sl].float().cpu().numpy())
    assert np.all(Tp[n:] == 0) and np.all(Tp[:, n:] == 0), "padded rows/columns of T' must be 0"
    Tp = Tp[:n, :n]
    worst["tp_relfro"] = max(worst["tp_relfro"], relfro(Tp, Tp_ref))
    kk, vv = kk[:n], vv[:n]
    worst["w_relfro"] = max(worst["w_relfro"], relfro(Tp @ (np.exp(G)[:, None] * kk), W_ref))
    worst["u_relfro"] = max(worst["u_relfro"], relfro(Tp @ vv, U_ref))


def check_chunks(dp, p, i, heads, chunks, report=None):
    """Stage-1 intermediates of the given chunks of sequence i and v-heads
    ``heads``, each against the oracle's stage-1 functions on that chunk's
    inputs alone (the intermediates depend on nothing else), so that chunks of
    the longest sequences can be checked without running the oracle over the
    whole sequence.  Returns a dict of worst errors."""
    heads_l = list(heads)
    norm = bool(getattr(dp, "flags", 0) & OPT_L2NORM_QK)
    arrs = seq_arrays(p, i, heads_l, normalize=norm)
    raw = seq_arrays(p, i, heads_l) if norm else arrs
    L = int(p.lengths[i])
    regions = {r: dp.region(r) for r in ("gc", "tp") + (("nrm",) if norm else ())}
    worst = dict(w_relfro=0.0, u_relfro=0.0, tp_relfro=0.0, gc_err=0.0, nrm_err=0.0)
    for c in chunks:
        a, b = 64 * c, min(L, 64 * c + 64)
        k_c, v_c, g_c, beta_c = arrs["k"][a:b], arrs["v"][a:b], arrs["g"][a:b], arrs["beta"][a:b]
        G = chunk_cumsum(g_c)
        Lm = gram_strict_lower(k_c, beta_c, G)
        Tp = ut_transform(Lm, beta_c)
        W, U = wy_solve(Lm, k_c, v_c, beta_c, G)
        for j, h in enumerate(heads_l):
            _compare_slot(regions, dp.slot(i, h, c), G[:, j], Tp[j], W[j], U[j], k_c[:, j], v_c[:, j], worst,
                          raw_qk=(raw["q"][a:b, j], raw["k"][a:b, j]) if norm else None)
    if report is not None:
        report.update(worst)
    return worst


def assert_within(worst, intermediates=False, entries=True):
    if os.environ.get("GDN_PARITY_VERBOSE"):
        print("worst errors:", {k: float("%.3g" % v) for k, v in worst.items()}, flush=True)
    if "o_maxabs" in worst:
        assert worst["o_maxabs"] <= TOL_O_MAXABS, worst
        assert worst["state_relfro"] <= TOL_STATE_RELFRO, worst
    if entries:
        assert worst["entry_maxabs"] <= TOL_ENTRY_MAXABS, worst
        assert worst["entry_relfro"] <= TOL_ENTRY_RELFRO, worst
    if intermediates:
        assert worst["gc_err"] <= 1e-4, worst
        assert worst.get("nrm_err", 0.0) <= TOL_NRM_REL, worst
        assert worst["tp_relfro"] <= TOL_TP_RELFRO, worst
        assert worst["w_relfro"] <= TOL_WU_RELFRO, worst
        assert worst["u_relfro"] <= TOL_WU_RELFRO, worst
