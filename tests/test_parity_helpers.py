"""The GPU tests' comparisons (tests/parity.py) on the CPU: a stand-in for the
device problem whose scratch holds the oracle's own gc, T' (as the bf16 hi +
lo pair) and row scales in the documented layout must pass, and one with a
planted mistake must not; likewise outputs and states.  No GPU is
involved."""

import numpy as np
import pytest
import torch

from oracle import l2_normalize
from oracle.chunked import chunk_cumsum, gram_strict_lower, ut_transform
from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64, make_problem
from parity import (_TP_S, _TP_T, OPT_L2NORM_QK, TOL_NRM_REL, TOL_TP_RELFRO, assert_within, check_chunks,
                    seq_arrays)


def _bf16_pair(x):
    """hi = bf16(x), lo = bf16(x - hi), as float32 values."""
    x = torch.from_numpy(np.asarray(x, np.float32))
    hi = x.to(torch.bfloat16).float()
    lo = (x - hi).to(torch.bfloat16).float()
    return hi.numpy(), lo.numpy()


class ScratchFromOracle:
    """Minimal stand-in for DeviceProblem: region() and slot() over scratch
    filled from the oracle (slots in [seq][v-head][chunk] order).  With
    ``norm`` the call is one with q/k normalisation: the oracle normalises q
    and k, and the scratch also holds the row scales."""

    def __init__(self, p, plant=None, norm=False):
        self.p = p
        self.flags = 0x1 | (OPT_L2NORM_QK if norm else 0)
        nv = p.nv
        slots = int(p.cu_chunks[-1]) * nv
        gc = np.zeros((slots, 64), np.float32)
        tp = np.zeros((slots, 2, 2560), np.float32)
        nrm = np.zeros((slots, 2, 64), np.float32)
        for i in range(p.nseq):
            arrs = seq_arrays(p, i, normalize=norm)
            raw = seq_arrays(p, i)
            L = int(p.lengths[i])
            for c in range(int(p.cu_chunks[i + 1] - p.cu_chunks[i])):
                a, b = 64 * c, min(L, 64 * c + 64)
                n = b - a
                G = chunk_cumsum(arrs["g"][a:b])
                Tp = ut_transform(gram_strict_lower(arrs["k"][a:b], arrs["beta"][a:b], G), arrs["beta"][a:b])
                for h in range(nv):
                    sl = self.slot(i, h, c)
                    gc[sl, :n] = G[:, h]
                    gc[sl, n:] = G[-1, h]
                    T = np.zeros((64, 64))
                    T[:n, :n] = Tp[h].T if plant == "transposed" else Tp[h]
                    tp[sl, 0], tp[sl, 1] = _bf16_pair(T[_TP_T, _TP_S])
                    for part, x in ((0, raw["k"][a:b, h]), (1, raw["q"][a:b, h])):
                        s = 1.0 / np.linalg.norm(x, axis=-1)
                        if plant == "squared_norm":
                            s = s * s
                        nrm[sl, part, :n] = s
                        nrm[sl, part, n:] = s[-1]
        self._r = dict(gc=torch.from_numpy(gc), tp=torch.from_numpy(tp), nrm=torch.from_numpy(nrm))

    def region(self, name):
        return self._r[name]

    def slot(self, i, h, c):
        chunk0 = int(self.p.cu_chunks[i])
        nch = int(self.p.cu_chunks[i + 1] - self.p.cu_chunks[i])
        return chunk0 * self.p.nv + h * nch + c


@pytest.fixture(scope="module")
def problem():
    return make_problem([200, 64, 131], nk=1, nv=2, seed=5)


def test_oracle_values_pass(problem):
    dp = ScratchFromOracle(problem)
    for i in range(problem.nseq):
        nch = int(problem.cu_chunks[i + 1] - problem.cu_chunks[i])
        w = check_chunks(dp, problem, i, range(problem.nv), range(nch))
        assert_within(w, intermediates=True, entries=False)
        # only the rounding of the bf16 hi + lo pair remains
        assert 0 < w["tp_relfro"] <= 2.0 ** -16


def test_planted_mistake_fails(problem):
    dp = ScratchFromOracle(problem, plant="transposed")
    w = check_chunks(dp, problem, 0, [0], [0, 1])
    assert w["tp_relfro"] > 10 * TOL_TP_RELFRO
    with pytest.raises(AssertionError):
        assert_within(w, intermediates=True, entries=False)


@pytest.fixture(scope="module")
def raw_problem():
    return make_problem([150, 64], nk=1, nv=2, seed=6, raw_qk=True)


def test_normalised_call_oracle_values_pass(raw_problem):
    """Raw q, k with the normalisation option: the oracle's T' of the
    normalised keys and the exact row scales pass."""
    dp = ScratchFromOracle(raw_problem, norm=True)
    for i in range(raw_problem.nseq):
        nch = int(raw_problem.cu_chunks[i + 1] - raw_problem.cu_chunks[i])
        w = check_chunks(dp, raw_problem, i, range(raw_problem.nv), range(nch))
        assert_within(w, intermediates=True, entries=False)
        assert w["nrm_err"] <= 1e-6


@pytest.mark.parametrize("plant", ["squared_norm", "transposed"])
def test_normalised_call_planted_mistakes_fail(raw_problem, plant):
    dp = ScratchFromOracle(raw_problem, plant=plant, norm=True)
    w = check_chunks(dp, raw_problem, 0, [0, 1], [0, 1, 2])
    with pytest.raises(AssertionError):
        assert_within(w, intermediates=True, entries=False)


def test_raw_problem_keys_are_not_unit(raw_problem):
    """The raw-q/k inputs really are off unit length (so the option matters)."""
    k = bf16_to_f64(raw_problem.k)
    assert np.abs(np.linalg.norm(k, axis=-1) - 1).min() > 1
    assert np.allclose(np.linalg.norm(l2_normalize(k), axis=-1), 1)


class ResultsFromOracle:
    """Stand-in for DeviceProblem's results: outputs, final states and entry
    states ([dv][dk], bf16) as the oracle's recurrence gives them, in the
    documented layouts; ``plant="state_t"`` stores each final state
    transposed, ``plant="entry_t"`` each entry state."""

    def __init__(self, p, plant=None):
        from oracle import gdn_recurrence
        self.p = p
        self._cu_chunks = p.cu_chunks
        nslots = int(self._cu_chunks[-1]) * p.nv
        self.out = np.zeros((p.n_tokens, p.nv, 128), np.float32)
        self.h = np.zeros((p.nseq, p.nv, 128, 128), np.float32)
        ent = torch.zeros((nslots, 128, 128), dtype=torch.bfloat16)
        cu = p.cu_seqlens
        for i in range(p.nseq):
            o, hf, e = gdn_recurrence(**seq_arrays(p, i))
            self.out[cu[i]:cu[i + 1]] = o
            self.h[i] = np.swapaxes(hf, 1, 2) if plant == "state_t" else hf
            for hh in range(p.nv):
                for c in range(e.shape[0]):
                    ec = e[c, hh] if plant == "entry_t" else e[c, hh].T
                    ent[self.slot(i, hh, c)] = torch.from_numpy(np.ascontiguousarray(ec).astype(np.float32))
        self._ent = ent

    def output_rows(self, a, b, heads):
        return self.out[a:b][:, list(heads)]

    def state_of(self, i):
        return self.h[i]

    def region(self, name):
        assert name == "s_entry"
        return self._ent

    def slot(self, i, h, c):
        chunk0 = int(self._cu_chunks[i])
        nch = int(self._cu_chunks[i + 1]) - chunk0
        return chunk0 * self.p.nv + h * nch + c


@pytest.mark.parametrize("chunked", [False, True])
def test_check_problem_passes_oracle_results(problem, chunked):
    from parity import check_problem
    w = check_problem(ResultsFromOracle(problem), problem, chunked=chunked)
    assert_within(w)
    # only the float32 / bf16 storage of the stand-in remains
    assert w["o_maxabs"] < 1e-5 and w["state_relfro"] < 1e-6 and w["entry_relfro"] <= 2.0 ** -8


def test_check_problem_rejects_transposed_state(problem):
    from parity import TOL_STATE_RELFRO, check_problem
    w = check_problem(ResultsFromOracle(problem, plant="state_t"), problem, seqs=[0], heads=[1])
    assert w["state_relfro"] > 10 * TOL_STATE_RELFRO
    with pytest.raises(AssertionError):
        assert_within(w)


def test_check_problem_rejects_transposed_entry_states(problem):
    """Entry states stored [dk][dv] instead of the documented [dv][dk] fail."""
    from parity import TOL_ENTRY_MAXABS, check_problem
    w = check_problem(ResultsFromOracle(problem, plant="entry_t"), problem, seqs=[0], heads=[1])
    assert w["entry_maxabs"] > TOL_ENTRY_MAXABS
    with pytest.raises(AssertionError):
        assert_within(w)
