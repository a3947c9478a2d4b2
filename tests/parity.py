"""Comparison of the GPU library with the oracle (helpers for the gpu tests).

Tolerances (written here once, used by every parity test):
  * outputs o (bf16): max |o_gpu - o_ref| <= 2e-2
  * final state (f32): relative Frobenius error <= 1e-3 per (sequence, head)
  * entry states (bf16): max abs <= 2e-2, relative Frobenius <= 4e-3
    (bf16 storage alone is ~2^-9 relative)
  * gc: |err| <= 1e-4 * (1 + |G|)   (64 float32 additions)
  * W, U (float32): relative Frobenius <= 1e-4 per slot (hi/lo bf16 products
    carry ~2^-17 relative error)
  * uc (bf16): relative Frobenius <= 8e-3 per slot
"""

import numpy as np

from oracle import gdn_chunked, gdn_recurrence, kv_head_map
from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64

TOL_O_MAXABS = 2e-2
TOL_STATE_RELFRO = 1e-3
TOL_ENTRY_MAXABS = 2e-2
TOL_ENTRY_RELFRO = 4e-3
TOL_WU_RELFRO = 1e-4
TOL_UC_RELFRO = 8e-3


def relfro(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def seq_arrays(p, i, heads=None):
    """Oracle inputs of sequence i restricted to v-heads ``heads``; the k-heads
    are selected with the documented grouping so the oracle sees nk = nv."""
    a, b = int(p.cu_seqlens[i]), int(p.cu_seqlens[i + 1])
    heads = list(range(p.nv)) if heads is None else list(heads)
    kap = kv_head_map(p.nk, p.nv)[heads]
    return dict(q=bf16_to_f64(p.q[a:b][:, kap]), k=bf16_to_f64(p.k[a:b][:, kap]),
                v=bf16_to_f64(p.v[a:b][:, heads]), g=p.g[a:b][:, heads].astype(np.float64),
                beta=p.beta[a:b][:, heads].astype(np.float64), h0=p.h0[i][heads].astype(np.float64))


def check_problem(dp, p, seqs=None, heads=None, intermediates=False, entries=True, report=None):
    """Run the oracle on (seqs x heads) and compare with what the GPU left in
    ``dp`` (output, final state, scratch).  Returns a dict of worst errors."""
    seqs = range(p.nseq) if seqs is None else seqs
    heads_l = list(range(p.nv)) if heads is None else list(heads)
    out = dp.output()
    state = dp.state()
    worst = dict(o_maxabs=0.0, state_relfro=0.0, entry_maxabs=0.0, entry_relfro=0.0,
                 w_relfro=0.0, u_relfro=0.0, uc_relfro=0.0, gc_err=0.0)
    regions = {}
    if entries or intermediates:
        regions["s_entry"] = dp.region("s_entry")
    if intermediates:
        for r in ("gc", "w", "u", "uc"):
            regions[r] = dp.region(r)
    for i in seqs:
        a = int(p.cu_seqlens[i])
        L = int(p.lengths[i])
        arrs = seq_arrays(p, i, heads_l)
        if intermediates:
            o_ref, h_ref, ent_ref, inter = gdn_chunked(**arrs, keep_intermediates=True)
        else:
            o_ref, h_ref, ent_ref = gdn_recurrence(**arrs)
        if L:
            o_gpu = out[a:a + L][:, heads_l]
            worst["o_maxabs"] = max(worst["o_maxabs"], float(np.abs(o_gpu - o_ref).max()))
        for j, h in enumerate(heads_l):
            e = relfro(state[i][h].astype(np.float64), h_ref[j])
            worst["state_relfro"] = max(worst["state_relfro"], e)
            for c in range(ent_ref.shape[0]):
                sl = dp.slot(i, h, c)
                if "s_entry" in regions:
                    s_gpu = regions["s_entry"][sl].float().cpu().numpy().astype(np.float64)
                    worst["entry_maxabs"] = max(worst["entry_maxabs"], float(np.abs(s_gpu - ent_ref[c, j]).max()))
                    worst["entry_relfro"] = max(worst["entry_relfro"], relfro(s_gpu, ent_ref[c, j]))
                if intermediates:
                    n = min(64, L - 64 * c)
                    d = inter[c]
                    gc_gpu = regions["gc"][sl].cpu().numpy().astype(np.float64)
                    G = d["gc"][:, j]
                    worst["gc_err"] = max(worst["gc_err"], float((np.abs(gc_gpu[:n] - G) / (1 + np.abs(G))).max()))
                    # rows past the end repeat the last value
                    worst["gc_err"] = max(worst["gc_err"], float(np.abs(gc_gpu[n:] - G[-1]).max(initial=0)))
                    w_gpu = regions["w"][sl].cpu().numpy().astype(np.float64)
                    u_gpu = regions["u"][sl].cpu().numpy().astype(np.float64)
                    worst["w_relfro"] = max(worst["w_relfro"], relfro(w_gpu[:n], d["W"][j]))
                    worst["u_relfro"] = max(worst["u_relfro"], relfro(u_gpu[:n], d["U"][j]))
                    assert np.all(w_gpu[n:] == 0) and np.all(u_gpu[n:] == 0), "padded W/U rows must be 0"
                    uc_gpu = regions["uc"][sl].float().cpu().numpy().astype(np.float64).T  # [t][dv]
                    worst["uc_relfro"] = max(worst["uc_relfro"], relfro(uc_gpu[:n], d["uc"][j]))
    if report is not None:
        report.update(worst)
    return worst


def assert_within(worst, intermediates=False, entries=True):
    assert worst["o_maxabs"] <= TOL_O_MAXABS, worst
    assert worst["state_relfro"] <= TOL_STATE_RELFRO, worst
    if entries:
        assert worst["entry_maxabs"] <= TOL_ENTRY_MAXABS, worst
        assert worst["entry_relfro"] <= TOL_ENTRY_RELFRO, worst
    if intermediates:
        assert worst["gc_err"] <= 1e-4, worst
        assert worst["w_relfro"] <= TOL_WU_RELFRO, worst
        assert worst["u_relfro"] <= TOL_WU_RELFRO, worst
        assert worst["uc_relfro"] <= TOL_UC_RELFRO, worst
