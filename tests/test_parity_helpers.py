"""The GPU tests' stage-1 comparison (tests/parity.py) on the CPU: a stand-in
for the device problem whose scratch holds the oracle's own gc, decays and T'
in the documented layout must pass, and one with a planted mistake in T' must
not.  No GPU is involved."""

import numpy as np
import pytest
import torch

from oracle.chunked import chunk_cumsum, gram_strict_lower, ut_transform
from linear_attention_ssm_chunk_amd.inputs import make_problem
from parity import _TP_S, _TP_T, TOL_TP_RELFRO, assert_within, check_chunks, seq_arrays


class ScratchFromOracle:
    """Minimal stand-in for DeviceProblem: region() and slot() over scratch
    filled from the oracle (slots in [seq][v-head][chunk] order)."""

    def __init__(self, p, plant=None):
        self.p = p
        nv = p.nv
        slots = int(p.cu_chunks[-1]) * nv
        gc = np.zeros((slots, 64), np.float32)
        dec = np.zeros((slots, 2, 64), np.float32)
        tp = np.zeros((slots, 2560), np.float16)
        for i in range(p.nseq):
            arrs = seq_arrays(p, i)
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
                    dec[sl, 0, :n] = np.exp(G[:, h])
                    dec[sl, 1, :n] = np.exp(G[-1, h] - G[:, h])
                    T = np.zeros((64, 64))
                    T[:n, :n] = Tp[h].T if plant == "transposed" else Tp[h]
                    tp[sl] = T[_TP_T, _TP_S].astype(np.float16)
        self._r = dict(gc=torch.from_numpy(gc), dec=torch.from_numpy(dec), tp=torch.from_numpy(tp))

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
        # only the float16 rounding of T' remains
        assert 0 < w["tp_relfro"] <= 2.0 ** -11


def test_planted_mistake_fails(problem):
    dp = ScratchFromOracle(problem, plant="transposed")
    w = check_chunks(dp, problem, 0, [0], [0, 1])
    assert w["tp_relfro"] > 10 * TOL_TP_RELFRO
    with pytest.raises(AssertionError):
        assert_within(w, intermediates=True, entries=False)


class ResultsFromOracle:
    """Stand-in for DeviceProblem's results: outputs, final states and entry
    states ([dv][dk], bf16) as the oracle's recurrence gives them, in the
    documented layouts; ``plant="state_t"`` stores each final state
    transposed."""

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
                    ent[self.slot(i, hh, c)] = torch.from_numpy(e[c, hh].T.astype(np.float32))
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
