"""gdn_prefill_noalloc, the entry point for callers that cannot allocate,
against gdn_prefill_ex on the same inputs, through the C ABI: outputs, final
states and entry states bit for bit the same (the same kernels, only the
intermediates live in the library's fixed array), on two calls in a row, the
second smaller, with and without entry states and q/k normalisation.  Sizes
beyond the fixed array are refused before anything touches the GPU."""

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from linear_attention_ssm_chunk_amd import binding as B  # noqa: E402
from linear_attention_ssm_chunk_amd import inputs as I  # noqa: E402
from parity import assert_within, check_problem  # noqa: E402

ENTRY, NORM = B.GDN_OPT_ENTRY_STATES, B.GDN_OPT_L2NORM_QK
NOALLOC_BYTES = 128 << 20  # GDN_NOALLOC_SCRATCH_BYTES


def _noalloc_fn():
    L = B.lib()
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.gdn_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(B.gdn_strides), ctypes.POINTER(B.gdn_varlen), ctypes.c_uint, vp]
    L.gdn_prefill_noalloc.restype = i32
    return L.gdn_prefill_noalloc


def _call_noalloc(dp, s_entry_out, stream):
    a = dp.args()
    vl = ctypes.byref(dp.varlen) if dp.varlen is not None else None
    return _noalloc_fn()(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], s_entry_out, dp.B, dp.T, dp.nk, dp.nv,
                         128, 128, ctypes.byref(dp.strides), vl, dp.flags, stream)


def test_sizes_beyond_the_array_are_refused_on_the_host():
    """B=4, T=8192, nv=32 needs 16384 slots of intermediates (about 172 MB): refused
    with GDN_ESCRATCH and a message, before any GPU call (pointers are fake)."""
    P = 0x7F0000000000
    st = B.gdn_strides(16 * 128, 32 * 128, 32)
    rc = _noalloc_fn()(P, P, P, P, P, P, 0, P, P, 4, 8192, 16, 32, 128, 128, ctypes.byref(st), None, 0, None)
    assert rc == B.GDN_ESCRATCH
    assert "fixed array" in B.gdn_last_error()
    rc = _noalloc_fn()(P, P, P, P, P, P, 0, P, None, 1, 64, 1, 1, 128, 128, ctypes.byref(st), None, ENTRY, None)
    assert rc == B.GDN_EINVAL and "s_entry_out" in B.gdn_last_error()


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [ENTRY, 0, ENTRY | NORM])
def test_noalloc_equals_prefill_ex_twice(flags):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_ssm_chunk_amd.device import DeviceProblem, current_stream_handle
    raw = bool(flags & NORM)
    cases = [
        # (lengths, nk, nv, kwargs): the second call is smaller than the first
        (I.make_problem([700, 1000, 333], nk=4, nv=8, seed=80, raw_qk=raw), dict(state="table", ragged=True)),
        (I.make_problem([150], nk=1, nv=2, seed=81, raw_qk=raw), {}),
    ]
    for p, kw in cases:
        print(f"[gpu] noalloc flags={flags} lengths={p.lengths} nk={p.nk} nv={p.nv} {kw}", flush=True)
        ref = DeviceProblem(p, flags=flags, **kw)
        ref.run()
        got = DeviceProblem(p, flags=flags, **kw)
        slots = int(p.cu_chunks[-1]) * p.nv
        ent = torch.empty((slots, 128, 128), dtype=torch.bfloat16, device="cuda") if flags & ENTRY else None
        got.out.fill_(0)
        rc = _call_noalloc(got, ent.data_ptr() if ent is not None else None, current_stream_handle())
        assert rc == B.GDN_OK, B.gdn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.out, ref.out)
        assert np.array_equal(got.state(), ref.state())
        if ent is not None:
            assert torch.equal(ent, ref.region("s_entry"))
        assert_within(check_problem(got, p, seqs=[0], entries=False))


@pytest.mark.gpu
def test_noalloc_under_graph_capture():
    """The call captured in a HIP graph (torch.cuda.graph) after one eager call
    on the device: three replays, with the state reset and the outputs
    cleared by eager work between them, each bit for bit equal to
    gdn_prefill_ex on the same inputs (outputs, final states, entry states)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_ssm_chunk_amd.device import DeviceProblem, current_stream_handle
    p = I.make_problem([700, 333], nk=2, nv=4, seed=83)
    print(f"[gpu] noalloc graph lengths={p.lengths}", flush=True)
    ref = DeviceProblem(p, flags=ENTRY, ragged=True)
    ref.run()
    torch.cuda.synchronize()
    got = DeviceProblem(p, flags=ENTRY, ragged=True)
    slots = int(p.cu_chunks[-1]) * p.nv
    ent = torch.empty((slots, 128, 128), dtype=torch.bfloat16, device="cuda")
    assert _call_noalloc(got, ent.data_ptr(), current_stream_handle()) == B.GDN_OK, B.gdn_last_error()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rc = _call_noalloc(got, ent.data_ptr(), current_stream_handle())
    assert rc == B.GDN_OK, B.gdn_last_error()
    for replay in range(3):
        got.reset_state()
        got.out.fill_(0)
        ent.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(got.out, ref.out), replay
        assert np.array_equal(got.state(), ref.state()), replay
        assert torch.equal(ent, ref.region("s_entry")), replay
