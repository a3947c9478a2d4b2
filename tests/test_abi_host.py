"""The C ABI on the host (CPU only): the library loads, exports every function
include/gdn_prefill.h declares, and rejects every malformed call by name
before touching the GPU."""

import os
import re

import pytest

from linear_attention_ssm_chunk_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_prefill.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(B.LIB_PATH):
        from linear_attention_ssm_chunk_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(gdn_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"gdn_prefill", "gdn_prefill_stage", "gdn_prefill_validate", "gdn_prefill_scratch_bytes",
            "gdn_prefill_scratch_layout", "gdn_varlen_check_host", "gdn_last_error", "gdn_prefill_ex",
            "gdn_prefill_stage_ex", "gdn_prefill_validate_ex", "gdn_prefill_scratch_bytes_ex",
            "gdn_prefill_scratch_layout_ex", "gdn_decode", "gdn_decode_validate"} <= set(names)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


# fake, well-aligned device addresses: validation never dereferences them
P = 0x7F0000000000


def good_args(**over):
    a = dict(q=P, k=P + 4096, v=P + 8192, g=P + 16384, beta=P + 16384 + 128, h_state=P + 2 ** 30,
             h_state_is_table=0, out=P + 2 ** 31, scratch=P + 2 ** 32, scratch_bytes=None,
             B=2, T=200, nk=2, nv=4, dk=128, dv=128, strides=(2 * 128, 4 * 128, 4), varlen=None)
    a.update(over)
    if a["scratch_bytes"] is None:
        a["scratch_bytes"] = B.gdn_prefill_scratch_bytes(a["B"], a["T"], max(a["nk"], 1), a["nv"], 128, 128,
                                                         a["varlen"]) or 1
    return a


def validate(**over):
    a = good_args(**over)
    rc = B.gdn_prefill_validate(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h_state"], a["h_state_is_table"],
                                a["out"], a["scratch"], a["scratch_bytes"], a["B"], a["T"], a["nk"], a["nv"],
                                a["dk"], a["dv"], a["strides"], a["varlen"])
    return rc, B.gdn_last_error()


def test_good_arguments_validate():
    rc, msg = validate()
    assert rc == B.GDN_OK and msg == ""


@pytest.mark.parametrize("over,code,needle", [
    (dict(dk=64), B.GDN_EUNSUPPORTED, "head size"),
    (dict(dv=256), B.GDN_EUNSUPPORTED, "head size"),
    (dict(nk=3), B.GDN_EINVAL, "GQA grouping"),
    (dict(nk=0), B.GDN_EINVAL, "head counts"),
    (dict(B=0), B.GDN_EINVAL, "B=0"),
    (dict(T=0), B.GDN_EINVAL, "T=0"),
    (dict(q=0), B.GDN_EINVAL, "null pointer"),
    (dict(beta=0), B.GDN_EINVAL, "null pointer"),
    (dict(h_state=0), B.GDN_EINVAL, "null pointer"),
    (dict(out=0), B.GDN_EINVAL, "null pointer"),
    (dict(scratch=0), B.GDN_EINVAL, "null pointer"),
    (dict(strides=None), B.GDN_EINVAL, "strides is required"),
    (dict(k=P + 4096 + 8), B.GDN_EINVAL, "16-byte aligned"),
    (dict(g=P + 2), B.GDN_EINVAL, "4-byte aligned"),
    (dict(scratch=P + 2 ** 32 + 16), B.GDN_EINVAL, "256-byte"),
    (dict(strides=(2 * 128 + 4, 512, 4)), B.GDN_EINVAL, "multiples of 8"),
    (dict(strides=(128, 512, 4)), B.GDN_EINVAL, "smaller than nk*128"),
    (dict(strides=(256, 256, 4)), B.GDN_EINVAL, "smaller than nv*128"),
    (dict(strides=(256, 512, 3)), B.GDN_EINVAL, "gb_row"),
    (dict(h_state_is_table=2), B.GDN_EINVAL, "h_state_is_table"),
    (dict(scratch_bytes=1024), B.GDN_ESCRATCH, "needed"),
])
def test_each_guard_rejects_by_name(over, code, needle):
    rc, msg = validate(**over)
    assert rc == code, msg
    assert needle in msg


def test_grid_extent_guards():
    """Sizes whose launches would overflow a 32-bit work-item count, or the
    int chunk count of the parameter block, are rejected before any launch."""
    # B x ceil(T/64) chunk slots beyond INT32_MAX
    rc, msg = validate(B=65535, T=2 ** 31 - 1)
    assert rc == B.GDN_EINVAL and "chunk slots" in msg, msg
    # one long sequence: 2^25 chunks x 4 heads x 64 lanes = 2^33 work-items in stage 1
    rc, msg = validate(B=1, T=2 ** 31 - 1)
    assert rc == B.GDN_EINVAL and "stage-1 grid" in msg, msg
    # stage 2 launches up to 2 workgroups x 512 lanes per chain: 65535 x 65
    # chains exceed 2^32 work-items, 65535 x 64 (2^32 - 2^16 x 1024) do not
    rc, msg = validate(B=65535, T=64, nk=65, nv=65, strides=(65 * 128, 65 * 128, 65))
    assert rc == B.GDN_EINVAL and "stage-2 grid" in msg, msg
    assert validate(B=65535, T=64, nk=64, nv=64, strides=(64 * 128, 64 * 128, 64))[0] == B.GDN_OK


def test_ragged_guards():
    vl = B.gdn_varlen(P + 64, P + 128, 3, 5)
    rc, msg = validate(varlen=vl, T=300, scratch_bytes=B.gdn_prefill_scratch_bytes(2, 300, 2, 4, 128, 128, vl))
    assert rc == B.GDN_OK, msg
    rc, msg = validate(varlen=B.gdn_varlen(0, P + 128, 3, 5), T=300)
    assert rc == B.GDN_EINVAL and "cu_seqlens and cu_chunks" in msg
    rc, msg = validate(varlen=B.gdn_varlen(P + 64, P + 128, 6, 5), T=300)
    assert rc == B.GDN_EINVAL and "max_chunks" in msg
    rc, msg = validate(varlen=B.gdn_varlen(P + 64, P + 128, 3, 4), T=300)
    assert rc == B.GDN_EINVAL and "cannot hold" in msg
    # every chunk holds a token: more chunks than tokens is a bad table
    rc, msg = validate(varlen=B.gdn_varlen(P + 64, P + 128, 3, 5), T=4)
    assert rc == B.GDN_EINVAL and "exceeds T" in msg


def test_ragged_call_without_tokens():
    """T == 0 allows NULL token pointers only with no chunks at all: a table
    that still claims chunks is rejected before anything could be launched on
    NULL pointers."""
    none = dict(q=0, k=0, v=0, g=0, beta=0, out=0, T=0)
    vl0 = B.gdn_varlen(P + 64, P + 128, 0, 0)
    rc, msg = validate(varlen=vl0, scratch_bytes=4096, **none)
    assert rc == B.GDN_OK, msg
    rc, msg = validate(varlen=B.gdn_varlen(P + 64, P + 128, 1, 1), scratch_bytes=1 << 20, **none)
    assert rc == B.GDN_EINVAL and "exceeds T" in msg


def test_flags_are_checked():
    a = good_args()
    args = [a[k] for k in ("q", "k", "v", "g", "beta", "h_state", "h_state_is_table", "out", "scratch",
                           "scratch_bytes", "B", "T", "nk", "nv", "dk", "dv", "strides", "varlen")]
    assert B.gdn_prefill_validate_ex(*args, B.GDN_OPT_ENTRY_STATES) == B.GDN_OK
    assert B.gdn_prefill_validate_ex(*args, 0) == B.GDN_OK
    assert B.gdn_prefill_validate_ex(*args, B.GDN_OPT_L2NORM_QK) == B.GDN_OK
    assert B.gdn_prefill_validate_ex(*args, 0x4) == B.GDN_EINVAL
    assert "flags=0x4" in B.gdn_last_error()
    # the normalisation region needs scratch of its own
    args[9] = B.gdn_prefill_scratch_bytes_ex(2, 200, 2, 4, 128, 128, None, 0)
    assert B.gdn_prefill_validate_ex(*args, 0) == B.GDN_OK
    assert B.gdn_prefill_validate_ex(*args, B.GDN_OPT_L2NORM_QK) == B.GDN_ESCRATCH
    assert B.gdn_prefill_scratch_bytes_ex(2, 200, 2, 4, 128, 128, None, 0x8) == 0


def test_prefill_rejects_without_touching_the_gpu():
    a = good_args(dk=64)
    with pytest.raises(B.GdnError) as e:
        B.gdn_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h_state"], 0, a["out"], a["scratch"],
                      a["scratch_bytes"], a["B"], a["T"], a["nk"], a["nv"], 64, 128, a["strides"], None, 0)
    assert e.value.code == B.GDN_EUNSUPPORTED
    with pytest.raises(B.GdnError) as e:
        B.gdn_prefill_stage(3, *[good_args()[k] for k in ("q", "k", "v", "g", "beta", "h_state",
                                                            "h_state_is_table", "out", "scratch",
                                                            "scratch_bytes", "B", "T", "nk", "nv", "dk",
                                                            "dv", "strides", "varlen")], 0)
    assert "stage=3" in str(e.value)


def test_scratch_layout_arithmetic():
    L = B.gdn_prefill_scratch_layout(4, 8192, 16, 32, 128, 128)
    chunks = 4 * 128
    slots = chunks * 32
    assert L.slots == slots and L.gc == 0 and L.flags == B.GDN_OPT_ENTRY_STATES
    assert L.tp == slots * 64 * 4
    assert L.nrm == B.GDN_NO_REGION
    assert L.s_entry == L.tp + slots * 2 * 2560 * 2
    assert L.total == L.s_entry + slots * 128 * 128 * 2
    # no entry states: gc and T' only; with normalisation the row scales follow T'
    L0 = B.gdn_prefill_scratch_layout_ex(4, 8192, 16, 32, 128, 128, None, 0)
    assert L0.s_entry == B.GDN_NO_REGION and L0.nrm == B.GDN_NO_REGION
    assert L0.total == L.s_entry
    Ln = B.gdn_prefill_scratch_layout_ex(4, 8192, 16, 32, 128, 128, None,
                                         B.GDN_OPT_L2NORM_QK | B.GDN_OPT_ENTRY_STATES)
    assert Ln.nrm == L.s_entry and Ln.s_entry == Ln.nrm + slots * 2 * 64 * 4
    assert Ln.total == Ln.s_entry + slots * 128 * 128 * 2
    assert B.gdn_prefill_scratch_bytes(2, 0, 2, 4, 128, 128, B.gdn_varlen(P, P, 0, 0)) == 256
    # partial last chunk: T = 200 -> 4 chunks
    assert B.gdn_prefill_scratch_layout(1, 200, 1, 1, 128, 128).slots == 4
    # ragged: total_chunks decides
    vl = B.gdn_varlen(P, P, 2, 7)
    assert B.gdn_prefill_scratch_layout(3, 0, 5, 5, 128, 128, vl).slots == 35
    assert B.gdn_prefill_scratch_bytes(1, 64, 1, 1, 64, 128) == 0
    assert B.gdn_prefill_scratch_bytes(1, 64, 3, 4, 128, 128) == 0


def test_varlen_host_check():
    assert B.gdn_varlen_check_host(3, 200, [0, 65, 65, 200], [0, 2, 2, 5], 3, 5) == B.GDN_OK
    assert B.gdn_varlen_check_host(3, 200, [0, 65, 65, 200], [0, 1, 1, 4], 3, 4) == B.GDN_EINVAL
    assert "ceil(len/64)" in B.gdn_last_error()
    assert B.gdn_varlen_check_host(3, 200, [0, 65, 60, 200], [0, 2, 2, 5], 3, 5) == B.GDN_EINVAL
    assert "decreases" in B.gdn_last_error()
    assert B.gdn_varlen_check_host(3, 200, [0, 65, 65, 200], [0, 2, 2, 5], 2, 5) == B.GDN_EINVAL
    assert B.gdn_varlen_check_host(3, 200, [0, 65, 65, 200], [0, 2, 2, 5], 3, 6) == B.GDN_EINVAL
    # the offsets must end at the call's token count
    assert B.gdn_varlen_check_host(3, 199, [0, 65, 65, 200], [0, 2, 2, 5], 3, 5) == B.GDN_EINVAL
    assert "cu_seqlens[B]=200 but T=199" in B.gdn_last_error()
    assert B.gdn_varlen_check_host(3, 201, [0, 65, 65, 200], [0, 2, 2, 5], 3, 5) == B.GDN_EINVAL
    # fewer than B + 1 offsets: refused before the library reads past them
    with pytest.raises(ValueError):
        B.gdn_varlen_check_host(4, 200, [0, 65, 65, 200], [0, 2, 2, 5], 3, 5)


def test_host_tensors_are_refused():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="device memory"):
        validate(q=torch.zeros(8, dtype=torch.bfloat16))


def decode_args(**over):
    a = dict(q=P, k=P + 4096, v=P + 8192, g=P + 16384, beta=P + 16384 + 128, h_state=P + 2 ** 30,
             h_state_is_table=0, out=P + 2 ** 31, B=3, nk=2, nv=4, dk=128, dv=128,
             strides=B.gdn_strides(2 * 128, 4 * 128, 4))
    a.update(over)
    return a


def decode_validate(**over):
    a = decode_args(**over)
    rc = B.gdn_decode_validate(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h_state"], a["h_state_is_table"],
                               a["out"], a["B"], a["nk"], a["nv"], a["dk"], a["dv"], a["strides"])
    return rc, B.gdn_last_error()


def test_decode_validation_names_the_guard():
    assert decode_validate()[0] == B.GDN_OK
    rc, msg = decode_validate(dk=64)
    assert rc == B.GDN_EUNSUPPORTED and "head size" in msg
    rc, msg = decode_validate(nk=3, nv=4)
    assert rc == B.GDN_EINVAL and "GQA" in msg
    rc, msg = decode_validate(B=0)
    assert rc == B.GDN_EINVAL and "B=0" in msg
    rc, msg = decode_validate(q=0)
    assert rc == B.GDN_EINVAL and "null pointer" in msg
    rc, msg = decode_validate(out=0)
    assert rc == B.GDN_EINVAL and "out" in msg
    rc, msg = decode_validate(k=P + 8)
    assert rc == B.GDN_EINVAL and "alignment" in msg
    rc, msg = decode_validate(h_state_is_table=2)
    assert rc == B.GDN_EINVAL and "h_state_is_table" in msg
    rc, msg = decode_validate(strides=B.gdn_strides(2 * 128 + 4, 4 * 128, 4))
    assert rc == B.GDN_EINVAL and "multiples of 8" in msg
    rc, msg = decode_validate(strides=B.gdn_strides(128, 4 * 128, 4))
    assert rc == B.GDN_EINVAL and "qk_row" in msg
    rc, msg = decode_validate(strides=B.gdn_strides(2 * 128, 4 * 128, 3))
    assert rc == B.GDN_EINVAL and "gb_row" in msg
    # a table of state pointers only needs 8-byte alignment
    assert decode_validate(h_state=P + 8, h_state_is_table=1)[0] == B.GDN_OK
    # 2^24 heads x 4 workgroups x 64 lanes = 2^32 work-items; one head fewer fits
    rc, msg = decode_validate(nk=1, nv=2 ** 24, strides=B.gdn_strides(128, 2 ** 31, 2 ** 24))
    assert rc == B.GDN_EINVAL and "decode grid" in msg, msg
    nv = 2 ** 24 - 1
    assert decode_validate(nk=1, nv=nv, strides=B.gdn_strides(128, nv * 128, nv))[0] == B.GDN_OK


def test_decode_flags_are_checked():
    """gdn_decode_validate_ex accepts q/k normalisation and nothing else (an
    entry-state bit means nothing for one token); gdn_decode_validate is the
    call with no flags."""
    a = decode_args()
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["h_state"], a["h_state_is_table"], a["out"], a["B"],
            a["nk"], a["nv"], a["dk"], a["dv"], a["strides"])
    assert B.gdn_decode_validate_ex(*args, 0) == B.GDN_OK
    assert B.gdn_decode_validate_ex(*args, B.GDN_OPT_L2NORM_QK) == B.GDN_OK
    for bad in (B.GDN_OPT_ENTRY_STATES, B.GDN_OPT_ENTRY_STATES | B.GDN_OPT_L2NORM_QK, 0x4, 0x80000000):
        assert B.gdn_decode_validate_ex(*args, bad) == B.GDN_EINVAL
        assert "flags" in B.gdn_last_error() and "GDN_OPT_L2NORM_QK" in B.gdn_last_error()
    # the other guards run as without flags
    bad_nv = dict(a, nv=5)
    args_bad = (bad_nv["q"], bad_nv["k"], bad_nv["v"], bad_nv["g"], bad_nv["beta"], bad_nv["h_state"], 0,
                bad_nv["out"], bad_nv["B"], bad_nv["nk"], bad_nv["nv"], 128, 128, bad_nv["strides"])
    assert B.gdn_decode_validate_ex(*args_bad, B.GDN_OPT_L2NORM_QK) == B.GDN_EINVAL
    assert "GQA" in B.gdn_last_error()
    with pytest.raises(B.GdnError) as e:
        B.gdn_decode_ex(*args, B.GDN_OPT_ENTRY_STATES, 0)
    assert e.value.code == B.GDN_EINVAL


def test_decode_rejects_without_touching_the_gpu():
    a = decode_args(nv=5)
    with pytest.raises(B.GdnError) as e:
        B.gdn_decode(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h_state"], 0, a["out"], a["B"], a["nk"],
                     a["nv"], 128, 128, a["strides"], 0)
    assert e.value.code == B.GDN_EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises: there is no
    other code path."""
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libgdn_prefill.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        B.gdn_prefill_scratch_bytes(1, 64, 1, 1, 128, 128)
    with pytest.raises(ImportError):
        B.gdn_decode_validate(P, P, P, P, P, P, 0, P, 1, 1, 1, 128, 128, B.gdn_strides(128, 128, 1))
