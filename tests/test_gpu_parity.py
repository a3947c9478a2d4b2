"""Parity of the HIP library with the oracle, on the GPU, through the C ABI.

Small problems (seconds of oracle time, several chunks and a ragged tail) are
compared element by element, intermediates included; the full-size workloads
run in the launch configuration bench.py times and are compared on sampled
(sequence, head) chains, each computed by the oracle in full.  Tolerances are
in tests/parity.py.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from linear_attention_ssm_chunk_amd import inputs as I  # noqa: E402
from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64  # noqa: E402
from parity import assert_within, check_chunks, check_problem, relfro  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_ssm_chunk_amd import binding
    binding.lib()  # fails loudly if the library is not built
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    return DeviceProblem


def run(DP, p, **kw):
    print(f"[gpu] lengths={p.lengths[:8]}{'...' if len(p.lengths) > 8 else ''} nk={p.nk} nv={p.nv} {kw}", flush=True)
    dp = DP(p, **kw)
    dp.run()
    torch.cuda.synchronize()
    return dp


# --------------------------------------------------------------------------
# small problems, full comparison


def test_workload1_tiny_full(dev):
    p = I.make_workload(1)
    dp = run(dev, p)
    w = check_problem(dp, p, intermediates=True)
    print(w)
    assert_within(w, intermediates=True)


@pytest.mark.parametrize("T", [200, 64, 1, 129])
def test_dense_gqa_ragged_tail(dev, T):
    p = I.make_problem([T, T], nk=2, nv=4, seed=100 + T)
    dp = run(dev, p)
    w = check_problem(dp, p, intermediates=True)
    print(w)
    assert_within(w, intermediates=True)


def test_gqa_ratio3_heads_distinguishable(dev):
    """nk=2, nv=6: each v-head must read k-head h*nk//nv (a swap fails)."""
    p = I.make_problem([150], nk=2, nv=6, seed=7)
    dp = run(dev, p)
    w = check_problem(dp, p, intermediates=True)
    assert_within(w, intermediates=True)


@pytest.mark.parametrize("case", [
    # (lengths, nk, nv, kwargs): chain counts (sequences x v-heads) that give
    # the spine 1, 2 and 4 strips per workgroup on a 256-CU MI355X (up to 32,
    # 33..64 and more than 64 chains), checked in full
    ([200, 131], 2, 8, {}),                                  # 16 chains
    ([130], 4, 40, {}),                                       # 40 chains, GQA 10
    ([1, 63, 64, 65, 200], 3, 12, dict(state="table", ragged=True)),  # 60 chains, GQA 4
    ([130, 130, 130], 8, 32, {}),                             # 96 chains
    ([5, 140, 64, 97], 4, 24, dict(state="table", ragged=True)),      # 96 chains, ragged
])
def test_every_strip_layout_in_full(dev, case):
    lens, nk, nv, kw = case
    p = I.make_problem(lens, nk=nk, nv=nv, seed=31 + nv)
    dp = run(dev, p, **kw)
    w = check_problem(dp, p, intermediates=True)
    print(f"{len(lens) * nv} chains: {w}", flush=True)
    assert_within(w, intermediates=True)


def test_ragged_with_state_table(dev):
    lens = [1, 64, 65, 130, 0, 77, 129, 3]
    p = I.make_problem(lens, nk=1, nv=2, seed=11)
    dp = run(dev, p, state="table", ragged=True)
    w = check_problem(dp, p, intermediates=True)
    print(w)
    assert_within(w, intermediates=True)
    # the empty sequence keeps its state bit for bit
    assert np.array_equal(dp.state()[4], p.h0[4])


def test_all_sequences_empty(dev):
    p = I.make_problem([0, 0], nk=1, nv=1, seed=12)
    dp = run(dev, p, ragged=True)
    assert np.array_equal(dp.state(), p.h0)


class _DistinctH0:
    """Initial states h0[i] = base[i % 61] * scale[i], scale[i] = float32(1 +
    i / nseq), distinct per sequence: built on the device in one pass rather
    than drawn and uploaded whole; h0[i] gives sequence i's on the host (the
    same float32 products)."""

    def __init__(self, nseq, nv, seed):
        self.base = 0.02 * np.random.default_rng(seed).standard_normal((61, nv, 128, 128), dtype=np.float32)
        self.scale = (1.0 + np.arange(nseq) / nseq).astype(np.float32)
        self.shape = (nseq, nv, 128, 128)

    def __getitem__(self, i):
        return self.base[i % 61] * self.scale[i]

    def to_torch(self, device):
        idx = torch.arange(self.shape[0], device=device) % 61
        return torch.from_numpy(self.base).to(device)[idx] * torch.from_numpy(self.scale).to(device)[:, None, None, None]


def _edge_sample(nseq, extra, n_random, seed):
    """The first and last 300 sequences, the indices in ``extra`` and
    ``n_random`` drawn at random."""
    drawn = np.random.default_rng(seed).choice(nseq, n_random, replace=False).tolist()
    return sorted(set(range(300)) | set(range(nseq - 300, nseq)) | set(extra) | set(drawn))


MAX_B = 65535  # the largest batch the boundary accepts (one grid row per sequence)


def test_largest_batch_ragged(dev):
    """B = 65535 ragged sequences, mostly of 0-3 tokens, with sequences of one
    to three chunks at both ends and in the middle.  Every empty sequence keeps
    its state bit for bit; a sample (both ends, the long ones, 1500 at random)
    against the oracle, entry states included."""
    lens = [(0, 1, 2, 3)[i % 4] for i in range(MAX_B)]
    long_ = {0: 130, 1: 65, 32768: 192, MAX_B - 3: 64, MAX_B - 1: 129}
    for i, L in long_.items():
        lens[i] = L
    p = I.make_problem(lens, nk=1, nv=1, seed=750, h0="none")
    p.h0 = _DistinctH0(MAX_B, 1, 751)
    print(f"[gpu] ragged B={MAX_B} nk=1 nv=1", flush=True)
    dp = dev(p, ragged=True)
    h_init = dp.h.clone()
    dp.run()
    torch.cuda.synchronize()
    empty = torch.from_numpy(np.flatnonzero(np.asarray(lens) == 0)).to(dp.h.device)
    assert torch.equal(dp.h[empty], h_init[empty])
    del h_init
    w = check_problem(dp, p, seqs=_edge_sample(MAX_B, long_, 1500, 752))
    print(w, flush=True)
    assert_within(w)


def test_largest_batch_decode(dev):
    """One decode step for B = 65535 sequences (GQA 2): a sample (both ends,
    1500 at random) against the oracle recurrence."""
    from oracle import gdn_recurrence
    from parity import seq_arrays
    p = I.make_problem([1] * MAX_B, nk=1, nv=2, seed=760, h0="none")
    p.h0 = _DistinctH0(MAX_B, 2, 761)
    print(f"[gpu] decode B={MAX_B} nk=1 nv=2", flush=True)
    dp = dev(p, ragged=False)
    dp.decode_step(0)
    torch.cuda.synchronize()
    out = dp.dec_out.float().cpu().numpy()
    cu = p.cu_seqlens
    o_err = s_err = 0.0
    for i in _edge_sample(MAX_B, (), 1500, 762):
        o_ref, h_ref, _ = gdn_recurrence(**seq_arrays(p, i, cu=cu))
        st = dp.state_of(i).astype(np.float64)
        o_err = max(o_err, float(np.abs(out[i] - o_ref[0]).max()))
        s_err = max(s_err, max(relfro(st[h], h_ref[h]) for h in range(p.nv)))
    print(f"decode B={MAX_B}: o_maxabs={o_err:.3g} state_relfro={s_err:.3g}", flush=True)
    assert o_err <= 2e-2 and s_err <= 1e-5


def test_offsets_past_2_31(dev):
    """One sequence of 140000 tokens (a ragged tail), nk=16, nv=64: the last
    heads' entry states lie past 2^31 elements into the scratch and the
    output's last rows past 2^31 bytes.  The last v-head (k-head 15, the far
    end of the scratch) against the oracle over the whole sequence, stage 1's
    intermediates at both ends and the middle of it."""
    p = I.make_problem([140000], nk=16, nv=64, seed=770)
    dp = run(dev, p)
    last = dp.slot(0, 63, 2187)
    assert last * 128 * 128 >= 2 ** 31 and 140000 * 64 * 128 * 2 >= 2 ** 31
    w = check_problem(dp, p, heads=[63])
    print(w, flush=True)
    assert_within(w)
    wc = check_chunks(dp, p, 0, [63], [0, 1093, 2187])
    print(wc, flush=True)
    assert_within(wc, intermediates=True, entries=False)


def test_packed_conv_layout_bit_identical(dev):
    p = I.make_problem([200, 200], nk=2, nv=6, seed=13)
    a = run(dev, p, layout="contiguous")
    b = run(dev, p, layout="conv")
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.h, b.h)
    assert torch.equal(a.scratch, b.scratch)


def test_state_table_equals_contiguous(dev):
    p = I.make_problem([100, 100, 100], nk=1, nv=2, seed=14)
    a = run(dev, p, state="contiguous")
    b = run(dev, p, state="table")
    assert torch.equal(a.out, b.out)
    assert np.array_equal(a.state(), b.state())


def test_rerun_is_byte_identical(dev):
    p = I.make_problem([300], nk=2, nv=4, seed=15)
    dp = run(dev, p)
    o1, h1 = dp.out.clone(), dp.h.clone()
    dp.reset_state()
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, dp.out) and torch.equal(h1, dp.h)


def test_two_streams_at_once(dev):
    """Two calls with their own outputs, states and scratch, enqueued back to
    back on two streams so that their kernels may run at the same time (which
    the header allows): each equals the same call run alone, bit for bit,
    outputs, final states and entry states, three times over."""
    pa = I.make_problem([4096], nk=2, nv=4, seed=91)
    pb = I.make_problem([1500, 700, 64], nk=4, nv=12, seed=92)  # one and two strips per workgroup
    refs = [run(dev, p, ragged=(p is pb)) for p in (pa, pb)]
    pair = [dev(p, ragged=(p is pb)) for p in (pa, pb)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        print(f"[gpu] two streams, pass {rep}", flush=True)
        for d in pair:
            d.reset_state()
            d.out.fill_(0)
            d.region("s_entry").fill_(0)
        torch.cuda.synchronize()
        for d, s in zip(pair, streams):
            d.run(s.cuda_stream)
        torch.cuda.synchronize()
        for d, r in zip(pair, refs):
            assert torch.equal(d.out, r.out) and torch.equal(d.h, r.h), rep
            assert torch.equal(d.region("s_entry"), r.region("s_entry")), rep


@pytest.mark.parametrize("flags,raw", [(0x1, False), (0x0, False), (0x3, True)])
def test_stages_in_order_equal_one_call(dev, flags, raw):
    """Stage 1 then stage 2 through gdn_prefill_stage_ex equal one
    gdn_prefill_ex call bit for bit -- outputs, final states and the whole
    scratch (intermediates, row scales, entry states) -- with and without
    entry states and q/k normalisation."""
    p = I.make_problem([190, 77], nk=2, nv=4, seed=16, raw_qk=raw)
    a = run(dev, p, flags=flags, ragged=True)
    b = dev(p, flags=flags, ragged=True)
    for st in (1, 2):
        b.run_stage(st)
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out) and torch.equal(a.h, b.h)
    assert torch.equal(a.scratch, b.scratch)


def test_split_resume_through_in_place_state(dev):
    """[0, T) at once equals [0, T1) then [T1, T) carried through h_state."""
    T, T1 = 320, 130
    p = I.make_problem([T], nk=1, nv=2, seed=17)
    whole = run(dev, p)
    first = I.make_problem([T1], 1, 2, seed=0)
    second = I.make_problem([T - T1], 1, 2, seed=0)
    for dst, sl in ((first, slice(0, T1)), (second, slice(T1, T))):
        dst.q, dst.k, dst.v, dst.g, dst.beta = p.q[sl], p.k[sl], p.v[sl], p.g[sl], p.beta[sl]
    first.h0 = p.h0
    a = run(dev, first)
    second.h0 = a.state()
    b = run(dev, second)
    out = np.concatenate([a.output(), b.output()])
    assert np.abs(out - whole.output()).max() <= 2e-2
    assert relfro(b.state().astype(np.float64), whole.state().astype(np.float64)) <= 1e-4


# --------------------------------------------------------------------------
# special inputs with closed-form answers


def _one_hot_keys(rng, N, nk):
    idx = rng.integers(0, 128, size=(N, nk))
    k = np.zeros((N, nk, 128), np.float32)
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    return I.f32_to_bf16_bits(k)


def test_q_equals_k_beta_one_returns_v(dev):
    """beta = 1, q = k, exactly unit keys: o_t = v_t for any g and h0."""
    rng = np.random.default_rng(21)
    p = I.make_problem([200], nk=1, nv=2, seed=21)
    p.k = _one_hot_keys(rng, 200, 1)
    p.q = p.k.copy()
    p.beta[:] = 1.0
    dp = run(dev, p)
    o = dp.output()
    err = np.abs(o - bf16_to_f64(p.v)).max()
    print("q=k beta=1 max err", err)
    assert err <= 2e-2
    assert_within(check_problem(dp, p))


def test_beta_zero_decays_only(dev):
    """beta = 0: o_t = exp(G_t) h0^T q_t, final state exp(sum g) h0.  The
    decay is slowed (g * 0.01) so the final state stays inside float32 range."""
    p = I.make_problem([150], nk=1, nv=2, seed=22)
    p.beta[:] = 0.0
    p.g *= np.float32(0.01)
    dp = run(dev, p)
    G = np.cumsum(p.g.astype(np.float64), axis=0)
    q = bf16_to_f64(p.q)[:, 0]
    expect = np.exp(G)[:, :, None] * np.einsum("hkd,tk->thd", p.h0[0].astype(np.float64), q)
    assert np.abs(dp.output() - expect).max() <= 2e-2
    hf = np.exp(G[-1])[:, None, None] * p.h0[0]
    assert relfro(dp.state()[0].astype(np.float64), hf) <= 1e-5


def test_one_hot_overwrite_no_decay(dev):
    """g = 0, beta = 1, one-hot keys: each token overwrites row pi(t) of h."""
    rng = np.random.default_rng(23)
    p = I.make_problem([150], nk=1, nv=1, seed=23)
    p.k = _one_hot_keys(rng, 150, 1)
    p.g[:] = 0.0
    p.beta[:] = 1.0
    dp = run(dev, p)
    h = p.h0[0, 0].astype(np.float64).copy()
    kk = bf16_to_f64(p.k)[:, 0]
    vv = bf16_to_f64(p.v)[:, 0]
    for t in range(150):
        h[np.argmax(kk[t])] = vv[t]
    assert relfro(dp.state()[0, 0].astype(np.float64), h) <= 1e-5
    assert_within(check_problem(dp, p))


def test_strong_forgetting(dev):
    p = I.make_problem([130], nk=1, nv=1, seed=24)
    p.g[:] = -80.0
    dp = run(dev, p)
    assert_within(check_problem(dp, p))


# --------------------------------------------------------------------------
# full-size workloads, sampled chains


@pytest.mark.slow
@pytest.mark.parametrize("index,samples", [
    (2, [(0, 0), (0, 17), (0, 31)]),
    (3, [(0, 0), (1, 9), (2, 22), (3, 31)]),
    (4, "per_seq"),
    (5, [(0, h) for h in (0, 16, 31, 47)]),
])
def test_full_workload_sampled(dev, index, samples):
    p = I.make_workload(index)
    kw = dict(layout="conv") if p.meta["layout"] == "conv" else {}
    if p.meta["layout"] == "varlen_table":
        kw = dict(state="table", ragged=True)
    dp = run(dev, p, **kw)
    out = dp.output()
    assert np.all(np.isfinite(out))
    if samples == "per_seq":
        samples = [(i, (5 * i + 3) % p.nv) for i in range(p.nseq)]
    worst = {}
    by_seq = {}
    for (i, h) in samples:
        by_seq.setdefault(i, []).append(h)
    for i, heads in by_seq.items():  # one oracle run per sequence over its sampled heads
        w = check_problem(dp, p, seqs=[i], heads=heads, entries=True)
        for key, val in w.items():
            worst[key] = max(worst.get(key, 0.0), val)
    print(f"workload {index}: {worst}", flush=True)
    assert_within(worst)
    # stage 1's intermediates of the first, a middle and the last chunk of
    # each sampled (sequence, head), at the full size
    inter = {}
    for (i, h) in samples:
        nch = int(p.cu_chunks[i + 1] - p.cu_chunks[i])
        w = check_chunks(dp, p, i, [h], sorted({0, nch // 2, nch - 1}))
        for key, val in w.items():
            inter[key] = max(inter.get(key, 0.0), val)
    print(f"workload {index} stage-1 chunks: {inter}", flush=True)
    assert_within(inter, intermediates=True, entries=False)


@pytest.mark.parametrize("index", [2, 3])
def test_workload_every_chain(dev, index):
    """The single-stream (T=4096, nv=32) and the batched (B=4, T=8192, nv=32,
    carried state) workloads at full size, in the launch the bench times:
    every (sequence, head) chain's outputs, final state and entry states
    against the oracle's chunk form."""
    p = I.make_workload(index)
    dp = run(dev, p)
    worst = {}
    for i in range(p.nseq):
        w = check_problem(dp, p, seqs=[i], chunked=True)
        print(f"sequence {i}: {w}", flush=True)
        for key, val in w.items():
            worst[key] = max(worst.get(key, 0.0), val)
    assert_within(worst)


@pytest.mark.parametrize("index", [6, 7])
def test_page_prompt_shapes_in_full(dev, index):
    """The prompt lengths page 1 profiles (1193 and 4593 tokens, ragged tails of
    41 and 49 tokens) at nk=16, nv=48 in the packed conv layout: every chain
    against the oracle's chunk form."""
    p = I.make_workload(index)
    dp = run(dev, p, layout="conv")
    w = check_problem(dp, p, chunked=True)
    print(f"workload {index}: {w}", flush=True)
    assert_within(w)


def test_ragged_workload_short_sequences_in_full(dev):
    """The ragged workload (8 sequences, state table) in the bench's launch:
    every head of each sequence shorter than 5000 tokens (6 of the 8; the two
    longest are sampled above) against the oracle's chunk form."""
    p = I.make_workload(4)
    dp = run(dev, p, state="table", ragged=True)
    short = [i for i in range(p.nseq) if p.lengths[i] < 5000]
    assert len(short) >= 4
    w = check_problem(dp, p, seqs=short, chunked=True)
    print(f"{len(short)} sequences x {p.nv} heads: {w}", flush=True)
    assert_within(w)


def test_slow_decay_long_carry(dev):
    """g * 0.01 keeps the state alive across many chunks, so a state that is
    not carried (or carried wrongly) between chunks shows in every output."""
    p = I.make_problem([700, 451], nk=2, nv=4, seed=25)
    p.g *= np.float32(0.01)
    dp = run(dev, p)
    w = check_problem(dp, p, intermediates=True)
    print(w)
    assert_within(w, intermediates=True)


# --------------------------------------------------------------------------
# decode: one recurrent step per sequence (gdn_decode)

def _decode_run(DP, p, steps, **kw):
    """Decode every token of p one step at a time; returns the outputs
    [T][B][nv][dv] (float) and the device problem (state after the last step)."""
    print(f"[gpu] decode lengths={p.lengths} nk={p.nk} nv={p.nv} {kw}", flush=True)
    dp = DP(p, ragged=False, **kw)
    outs = []
    for t in range(steps):
        dp.decode_step(t)
        torch.cuda.synchronize()
        outs.append(dp.dec_out.float().cpu().numpy())
    return np.stack(outs), dp


def _oracle_steps(p):
    """Oracle outputs [T][B][nv][dv] and final states of every sequence."""
    from parity import seq_arrays
    from oracle import gdn_recurrence
    T = p.lengths[0]
    o = np.zeros((T, p.nseq, p.nv, 128))
    hs = []
    for i in range(p.nseq):
        oi, hi, _ = gdn_recurrence(**seq_arrays(p, i))
        o[:, i] = oi
        hs.append(hi)
    return o, np.stack(hs)


@pytest.mark.parametrize("nk,nv", [(2, 6), (1, 1)])
def test_decode_one_token(dev, nk, nv):
    p = I.make_problem([1] * 5, nk=nk, nv=nv, seed=700 + nv)
    out, dp = _decode_run(dev, p, 1)
    o_ref, h_ref = _oracle_steps(p)
    assert np.abs(out - o_ref).max() <= 2e-2
    st = dp.state().astype(np.float64)
    assert max(relfro(st[i, h], h_ref[i, h]) for i in range(p.nseq) for h in range(p.nv)) <= 1e-5


def test_decode_steps_state_table_conv(dev):
    """Nine decode steps in a row on the packed conv layout with a state
    table: outputs at every step and the final state against the oracle."""
    p = I.make_problem([9] * 3, nk=1, nv=3, seed=710)
    out, dp = _decode_run(dev, p, 9, layout="conv", state="table")
    o_ref, h_ref = _oracle_steps(p)
    assert np.abs(out - o_ref).max() <= 2e-2
    st = dp.state().astype(np.float64)
    assert max(relfro(st[i, h], h_ref[i, h]) for i in range(p.nseq) for h in range(p.nv)) <= 1e-5


def test_decode_layouts_bit_identical(dev):
    p = I.make_problem([4] * 2, nk=2, nv=4, seed=720)
    a_out, a = _decode_run(dev, p, 4)
    b_out, b = _decode_run(dev, p, 4, layout="conv", state="table")
    assert np.array_equal(a_out, b_out) and np.array_equal(a.state(), b.state())


def test_decode_beta_zero_only_decays(dev):
    """beta = 0: h <- exp(g) h exactly (one float32 product), o = exp(g) h^T q."""
    p = I.make_problem([1] * 3, nk=1, nv=2, seed=730)
    p.beta[:] = 0
    out, dp = _decode_run(dev, p, 1)
    a = np.exp(p.g.astype(np.float64))  # [B][nv]
    want = (a[:, :, None, None] * p.h0.astype(np.float64)).astype(np.float32)
    assert np.abs(dp.state() - want).max() <= 1e-6 * np.abs(want).max()
    o_ref, _ = _oracle_steps(p)
    assert np.abs(out - o_ref).max() <= 2e-2


def test_decode_bench_batch_in_full(dev):
    """The decode the bench times (256 sequences, nk=16, nv=32, carried state,
    the same token applied step after step): every sequence and head after
    one step and after a second, against the oracle recurrence run over the
    token once and twice."""
    from oracle import gdn_recurrence
    from parity import seq_arrays
    p = I.make_problem([1] * 256, nk=16, nv=32, seed=6)
    print("[gpu] decode B=256 nk=16 nv=32, two steps", flush=True)
    dp = dev(p, ragged=False)
    twice = I.Problem([2] * 256, p.nk, p.nv, np.repeat(p.q, 2, axis=0), np.repeat(p.k, 2, axis=0),
                      np.repeat(p.v, 2, axis=0), np.repeat(p.g, 2, axis=0), np.repeat(p.beta, 2, axis=0),
                      p.h0, p.seed)
    cu1, cu2 = p.cu_seqlens, twice.cu_seqlens
    for step, (prob, cu) in enumerate(((p, cu1), (twice, cu2)), start=1):
        dp.decode_step(0)
        torch.cuda.synchronize()
        out = dp.dec_out.float().cpu().numpy()
        st = dp.state()
        o_err = s_err = 0.0
        for i in range(256):
            o_ref, h_ref, _ = gdn_recurrence(**seq_arrays(prob, i, cu=cu))
            o_err = max(o_err, float(np.abs(out[i] - o_ref[-1]).max()))
            s_err = max(s_err, max(relfro(st[i, h].astype(np.float64), h_ref[h]) for h in range(p.nv)))
        print(f"decode step {step}: o_maxabs={o_err:.3g} state_relfro={s_err:.3g}", flush=True)
        assert o_err <= 2e-2 and s_err <= 1e-5


def test_prefill_then_decode_continues_the_sequence(dev):
    """Prefill of 130 tokens (ragged chunk tail) leaves the state in place;
    decoding token 131 from it matches the oracle over all 131 tokens."""
    from parity import seq_arrays
    from oracle import gdn_recurrence
    T = 131
    full = I.make_problem([T] * 2, nk=2, nv=4, seed=740)
    rows = np.concatenate([np.arange(i * T, i * T + T - 1) for i in range(2)])
    last = np.array([i * T + T - 1 for i in range(2)])
    pre = I.Problem([T - 1] * 2, full.nk, full.nv, full.q[rows], full.k[rows], full.v[rows], full.g[rows],
                    full.beta[rows], full.h0.copy(), full.seed)
    one = I.Problem([1] * 2, full.nk, full.nv, full.q[last], full.k[last], full.v[last], full.g[last],
                    full.beta[last], full.h0.copy(), full.seed)
    dp = run(dev, pre)
    dd = dev(one, ragged=False)
    dd.h.copy_(dp.h)  # the prefill's final state, in place for the next token
    dd.decode_step(0)
    torch.cuda.synchronize()
    out = dd.dec_out.float().cpu().numpy()
    st = dd.state().astype(np.float64)
    for i in range(2):
        o_ref, h_ref, _ = gdn_recurrence(**seq_arrays(full, i))
        assert np.abs(out[i] - o_ref[-1]).max() <= 2e-2
        assert max(relfro(st[i, h], h_ref[h]) for h in range(full.nv)) <= 1e-3
