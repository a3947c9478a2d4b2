"""ctypes binding of libgdn_prefill.so (include/gdn_prefill.h).

Argument marshalling only: every function here converts its arguments to C
types and calls the function of the same name in the library.  Pointer
arguments take an int (a device address) or a tensor in device memory (an
object with ``data_ptr()``; one in host memory raises ValueError).  The library must have been built
(``python -m linear_attention_ssm_chunk_amd.build``); if it is missing, loading
fails with an error -- there is no other code path.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_prefill.so")

GDN_OK = 0
GDN_EINVAL = -1
GDN_EUNSUPPORTED = -2
GDN_ESCRATCH = -3
GDN_EHIP = -4
GDN_CHUNK = 64
GDN_HEAD_DIM = 128
GDN_OPT_ENTRY_STATES = 0x1
GDN_OPT_L2NORM_QK = 0x2
GDN_NO_REGION = ctypes.c_size_t(-1).value


class gdn_strides(ctypes.Structure):
    _fields_ = [("qk_row", ctypes.c_int64), ("v_row", ctypes.c_int64), ("gb_row", ctypes.c_int64)]


class gdn_varlen(ctypes.Structure):
    _fields_ = [("cu_seqlens", ctypes.c_void_p), ("cu_chunks", ctypes.c_void_p),
                ("max_chunks", ctypes.c_int32), ("total_chunks", ctypes.c_int32)]


class gdn_scratch_layout(ctypes.Structure):
    _fields_ = [("gc", ctypes.c_size_t), ("tp", ctypes.c_size_t), ("nrm", ctypes.c_size_t),
                ("s_entry", ctypes.c_size_t), ("total", ctypes.c_size_t),
                ("slots", ctypes.c_int64), ("flags", ctypes.c_uint)]


class GdnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gdn error {code}: {msg}")
        self.code = code


_lib = None


def load(path=None):
    """Load the library from ``path`` (default LIB_PATH; bench.py's section-stamp
    profiling loads libgdn_prefill_stamps.so this way before anything else).
    Once a library is loaded, every call goes to it."""
    global _lib
    if _lib is None:
        path = LIB_PATH if path is None else path
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run python -m linear_attention_ssm_chunk_amd.build")
        _lib = _declare(ctypes.CDLL(path))
    return _lib


def lib():
    """The loaded library (loaded on first use)."""
    return load()


def _declare(L):
    """Argument and result types of every exported function."""
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint
    common = [vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, i32, i32, i32, i32, i32, i32,
              ctypes.POINTER(gdn_strides), ctypes.POINTER(gdn_varlen)]
    L.gdn_prefill.argtypes = common + [vp]
    L.gdn_prefill.restype = i32
    L.gdn_prefill_ex.argtypes = common + [u32, vp]
    L.gdn_prefill_ex.restype = i32
    L.gdn_prefill_stage.argtypes = [i32] + common + [vp]
    L.gdn_prefill_stage.restype = i32
    L.gdn_prefill_stage_ex.argtypes = [i32] + common + [u32, vp]
    L.gdn_prefill_stage_ex.restype = i32
    L.gdn_prefill_validate.argtypes = common
    L.gdn_prefill_validate.restype = i32
    L.gdn_prefill_validate_ex.argtypes = common + [u32]
    L.gdn_prefill_validate_ex.restype = i32
    dims = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(gdn_varlen)]
    L.gdn_prefill_scratch_bytes.argtypes = dims
    L.gdn_prefill_scratch_bytes.restype = sz
    L.gdn_prefill_scratch_bytes_ex.argtypes = dims + [u32]
    L.gdn_prefill_scratch_bytes_ex.restype = sz
    L.gdn_prefill_scratch_layout.argtypes = dims + [ctypes.POINTER(gdn_scratch_layout)]
    L.gdn_prefill_scratch_layout.restype = i32
    L.gdn_prefill_scratch_layout_ex.argtypes = dims + [u32, ctypes.POINTER(gdn_scratch_layout)]
    L.gdn_prefill_scratch_layout_ex.restype = i32
    L.gdn_varlen_check_host.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                        ctypes.c_int32, ctypes.c_int32]
    L.gdn_varlen_check_host.restype = i32
    dec = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, ctypes.POINTER(gdn_strides)]
    L.gdn_decode.argtypes = dec + [vp]
    L.gdn_decode.restype = i32
    L.gdn_decode_ex.argtypes = dec + [u32, vp]
    L.gdn_decode_ex.restype = i32
    L.gdn_decode_validate.argtypes = dec
    L.gdn_decode_validate.restype = i32
    L.gdn_decode_validate_ex.argtypes = dec + [u32]
    L.gdn_decode_validate_ex.restype = i32
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    return L


def _ptr(x):
    """Device address of x.  A tensor in host memory is refused here: the
    kernels would dereference its address on the GPU."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        if getattr(x, "is_cuda", True) is not True:
            raise ValueError(f"tensor on {x.device}: every pointer argument must be in device memory")
        return x.data_ptr()
    return int(x)


def _strides(s):
    if s is None or isinstance(s, gdn_strides):
        return s
    return gdn_strides(*s)


def _varlen(v):
    if v is None or isinstance(v, gdn_varlen):
        return v
    cu_s, cu_c, mx, tot = v
    return gdn_varlen(_ptr(cu_s), _ptr(cu_c), int(mx), int(tot))


def _ref(struct):
    return ctypes.byref(struct) if struct is not None else None


def gdn_last_error():
    return lib().gdn_last_error().decode()


def _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
            B, T, nk, nv, dk, dv, strides, varlen):
    st, vl = _strides(strides), _varlen(varlen)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h_state), int(h_state_is_table),
            _ptr(out), _ptr(scratch), int(scratch_bytes), B, T, nk, nv, dk, dv, _ref(st), _ref(vl))
    return args, (st, vl)


def gdn_prefill(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                B, T, nk, nv, dk, dv, strides, varlen, stream):
    """Enqueue the prefill on ``stream`` (a hipStream_t as int).  Raises
    GdnError on a nonzero return."""
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    rc = lib().gdn_prefill(*args, ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_prefill_ex(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                   B, T, nk, nv, dk, dv, strides, varlen, flags, stream):
    """gdn_prefill with GDN_OPT_* flags.  Raises GdnError on a nonzero return."""
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    rc = lib().gdn_prefill_ex(*args, int(flags), ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_prefill_stage(stage, q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                      B, T, nk, nv, dk, dv, strides, varlen, stream):
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    rc = lib().gdn_prefill_stage(int(stage), *args, ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_prefill_stage_ex(stage, q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen, flags, stream):
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    rc = lib().gdn_prefill_stage_ex(int(stage), *args, int(flags), ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_prefill_validate(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen):
    """Return code of the pure host validation (no exception)."""
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    return lib().gdn_prefill_validate(*args)


def gdn_prefill_validate_ex(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                            B, T, nk, nv, dk, dv, strides, varlen, flags):
    args, keep = _common(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes,
                         B, T, nk, nv, dk, dv, strides, varlen)
    return lib().gdn_prefill_validate_ex(*args, int(flags))


def gdn_prefill_scratch_bytes(B, T, nk, nv, dk, dv, varlen=None):
    vl = _varlen(varlen)
    return lib().gdn_prefill_scratch_bytes(B, T, nk, nv, dk, dv, _ref(vl))


def gdn_prefill_scratch_bytes_ex(B, T, nk, nv, dk, dv, varlen=None, flags=GDN_OPT_ENTRY_STATES):
    vl = _varlen(varlen)
    return lib().gdn_prefill_scratch_bytes_ex(B, T, nk, nv, dk, dv, _ref(vl), int(flags))


def gdn_prefill_scratch_layout(B, T, nk, nv, dk, dv, varlen=None):
    vl = _varlen(varlen)
    out = gdn_scratch_layout()
    rc = lib().gdn_prefill_scratch_layout(B, T, nk, nv, dk, dv, _ref(vl), ctypes.byref(out))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return out


def gdn_prefill_scratch_layout_ex(B, T, nk, nv, dk, dv, varlen=None, flags=GDN_OPT_ENTRY_STATES):
    vl = _varlen(varlen)
    out = gdn_scratch_layout()
    rc = lib().gdn_prefill_scratch_layout_ex(B, T, nk, nv, dk, dv, _ref(vl), int(flags), ctypes.byref(out))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return out


def gdn_varlen_check_host(B, T, cu_seqlens, cu_chunks, max_chunks, total_chunks):
    """Check host copies of the ragged offsets (sequences of ints) for a call
    with T tokens in all."""
    if len(cu_seqlens) < B + 1 or len(cu_chunks) < B + 1:
        raise ValueError(f"offsets: {len(cu_seqlens)} and {len(cu_chunks)} entries given, B + 1 = {B + 1} needed")
    a = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    b = (ctypes.c_int32 * len(cu_chunks))(*[int(x) for x in cu_chunks])
    return lib().gdn_varlen_check_host(B, int(T), a, b, int(max_chunks), int(total_chunks))


def _decode_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides):
    st = _strides(strides)
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h_state), int(h_state_is_table), _ptr(out),
            B, nk, nv, dk, dv, _ref(st)), st


def gdn_decode(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, stream):
    """Enqueue one recurrent step per sequence on ``stream``.  Raises GdnError on
    a nonzero return."""
    args, keep = _decode_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides)
    rc = lib().gdn_decode(*args, ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_decode_ex(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, flags, stream):
    """gdn_decode with GDN_OPT_* flags (GDN_OPT_L2NORM_QK only).  Raises
    GdnError on a nonzero return."""
    args, keep = _decode_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides)
    rc = lib().gdn_decode_ex(*args, int(flags), ctypes.c_void_p(int(stream)))
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_decode_validate(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides):
    """Return code of the decode's host validation (no exception)."""
    args, keep = _decode_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides)
    return lib().gdn_decode_validate(*args)


def gdn_decode_validate_ex(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, flags):
    """Return code of gdn_decode_ex's host validation (no exception)."""
    args, keep = _decode_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides)
    return lib().gdn_decode_validate_ex(*args, int(flags))
