"""Seeded synthetic inputs for the chunked gated-delta-rule prefill.

This module draws random inputs and packs them into the memory layouts the
library accepts.  It holds none of the method's arithmetic; it is the one
module that both the oracle side (tests, bench cpu_baseline) and the GPU side
use, and it imports neither.

Recipe (fixed, documented in the design notes):
  * ragged workload: sequence lengths from ``numpy.random.default_rng(seed)``;
  * ``numpy.random.SeedSequence(seed).spawn(6)``: one stream per array, in the
    order q, k, v, g, beta, h0; per-token arrays are drawn in blocks of 4096
    tokens, block b from the b-th child of the array's stream (so blocks can
    be drawn in parallel and the result does not depend on thread count).
  * q, k ~ N(0, 1) float32, L2-normalised per (token, head) 128-vector in
    float32, then rounded to bf16 (round-to-nearest-even); v ~ N(0, 1) -> bf16.
    With ``raw_qk`` q and k are left as drawn (N(0, 1) -> bf16), for calls
    that normalise them inside the library.
  * g = -softplus(N(0, 1)) float32 (via logaddexp); beta = sigmoid(N(0, 1))
    float32.
  * h0 ~ N(0, 0.02^2) float32 where the workload has a carried state, else 0.

bf16 values are kept as ``uint16`` bit patterns; ``bf16_to_f64`` widens them
exactly.
"""

from dataclasses import dataclass, field

import numpy as np

CHUNK = 64
HEAD_DIM = 128


# ----------------------------------------------------------------------------
# bf16 helpers (bit patterns in uint16)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------
# workloads


WORKLOADS = {
    1: dict(name="tiny_T256", B=1, T=256, nk=1, nv=1, h0="zeros", layout="contiguous"),
    2: dict(name="single_stream_T4096", B=1, T=4096, nk=16, nv=32, h0="zeros", layout="contiguous"),
    3: dict(name="batched_B4_T8192_carried", B=4, T=8192, nk=16, nv=32, h0="normal",
            layout="contiguous", entry_states=True),
    4: dict(name="ragged_varlen_8seq", nseq=8, nk=16, nv=32, h0="normal", layout="varlen_table"),
    5: dict(name="long_packed_T65536", B=1, T=65536, nk=16, nv=48, h0="normal", layout="conv"),
    # the prompt lengths of the prefills page 1 profiles (its tensor-core spine
    # comment), at the head counts of workload 5: for setting the per-chunk
    # spine cost beside the page's, not graded workloads
    6: dict(name="page_prompt_T1193", B=1, T=1193, nk=16, nv=48, h0="zeros", layout="conv"),
    7: dict(name="page_prompt_T4593", B=1, T=4593, nk=16, nv=48, h0="zeros", layout="conv"),
}


def ragged_lengths(seed, nseq=8, lo=1, hi=16384, target=32768, tol=0.10):
    """Lengths for the ragged workload: ``nseq`` draws uniform in [lo, hi],
    none a multiple of 64, summing to ``target`` within ``tol``.  The first
    seed >= ``seed`` whose draw qualifies is used.  Returns (lengths, seed_used)."""
    s = seed
    while True:
        rng = np.random.default_rng(s)
        L = rng.integers(lo, hi + 1, size=nseq)
        if np.all(L % CHUNK != 0) and abs(int(L.sum()) - target) <= tol * target:
            return [int(x) for x in L], s
        s += 1


@dataclass
class Problem:
    """Canonical arrays of one synthetic problem (all sequences packed along
    the token axis)."""
    lengths: list
    nk: int
    nv: int
    q: np.ndarray          # uint16 bf16 bits [N, nk, 128]
    k: np.ndarray          # uint16 bf16 bits [N, nk, 128]
    v: np.ndarray          # uint16 bf16 bits [N, nv, 128]
    g: np.ndarray          # float32 [N, nv]
    beta: np.ndarray       # float32 [N, nv]
    h0: np.ndarray         # float32 [nseq, nv, 128, 128]  ([dk][dv])
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def n_tokens(self):
        return int(sum(self.lengths))

    @property
    def nseq(self):
        return len(self.lengths)

    @property
    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def cu_chunks(self):
        n = [-(-L // CHUNK) for L in self.lengths]
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)


BLOCK = 4096  # tokens per independent random stream


def _blocks(N):
    return [(a, min(N, a + BLOCK)) for a in range(0, N, BLOCK)] or [(0, 0)]


def _fill(seed_seq, N, fn, pool):
    """Concatenate fn(rng, rows) over token blocks, block b drawn from the
    b-th child of ``seed_seq`` (so the result does not depend on threads)."""
    blocks = _blocks(N)
    kids = seed_seq.spawn(len(blocks))
    parts = list(pool.map(lambda ab: fn(np.random.default_rng(kids[ab[0]]), ab[1][1] - ab[1][0]),
                          enumerate(blocks)))
    return np.concatenate(parts, axis=0)


def _unit_rows_bf16(rng, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    x /= np.linalg.norm(x, axis=-1, keepdims=True).astype(np.float32)
    return f32_to_bf16_bits(x)


def _raw_rows_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_problem(lengths, nk, nv, seed, h0="normal", raw_qk=False):
    """Draw q, k, v, g, beta, h0 for the given sequence lengths.

    ``SeedSequence(seed).spawn(6)`` gives one stream per array in the order q,
    k, v, g, beta, h0; the per-token arrays are drawn in blocks of 4096 tokens,
    block b from child b of the array's stream.  ``raw_qk``: q and k as drawn,
    not normalised."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    N = int(sum(lengths))
    ss = np.random.SeedSequence(seed).spawn(6)
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as pool:
        rows = _raw_rows_bf16 if raw_qk else _unit_rows_bf16
        q = _fill(ss[0], N, lambda r, n: rows(r, (n, nk, HEAD_DIM)), pool)
        k = _fill(ss[1], N, lambda r, n: rows(r, (n, nk, HEAD_DIM)), pool)
        v = _fill(ss[2], N, lambda r, n: f32_to_bf16_bits(r.standard_normal((n, nv, HEAD_DIM), dtype=np.float32)),
                  pool)
        g = _fill(ss[3], N, lambda r, n: (-np.logaddexp(np.float32(0), r.standard_normal((n, nv), dtype=np.float32))
                                          ).astype(np.float32), pool)
        beta = _fill(ss[4], N, lambda r, n: (1.0 / (1.0 + np.exp(-r.standard_normal((n, nv), dtype=np.float32)))
                                             ).astype(np.float32), pool)
    nseq = len(lengths)
    if h0 == "normal":
        h = (0.02 * np.random.default_rng(ss[5]).standard_normal((nseq, nv, HEAD_DIM, HEAD_DIM),
                                                                 dtype=np.float32)).astype(np.float32)
    elif h0 == "none":  # the caller sets p.h0
        h = None
    else:
        h = np.zeros((nseq, nv, HEAD_DIM, HEAD_DIM), dtype=np.float32)
    return Problem(list(lengths), nk, nv, q, k, v, g, beta, h, seed)


def make_workload(index, seed=None, raw_qk=False):
    """The synthetic problem of workload ``index`` (1..5) with seed = index
    unless given.  The ragged workload searches seeds from the base seed.
    ``raw_qk``: q and k left unnormalised (for calls that normalise them)."""
    w = WORKLOADS[index]
    seed = index if seed is None else seed
    if "nseq" in w:
        lengths, used = ragged_lengths(seed, w["nseq"])
        p = make_problem(lengths, w["nk"], w["nv"], used, w["h0"], raw_qk=raw_qk)
        p.meta["length_seed"] = used
    else:
        p = make_problem([w["T"]] * w["B"], w["nk"], w["nv"], seed, w["h0"], raw_qk=raw_qk)
    p.meta["raw_qk"] = raw_qk
    p.meta.update(w)
    p.meta["index"] = index
    return p


# ----------------------------------------------------------------------------
# layouts: host buffers in the shapes the library reads


def pack_contiguous(p):
    """Separate contiguous buffers: q, k [N][nk][128], v [N][nv][128], g, beta
    [N][nv].  Strides are per token row, in elements."""
    return dict(q=np.ascontiguousarray(p.q), k=np.ascontiguousarray(p.k),
                v=np.ascontiguousarray(p.v), g=np.ascontiguousarray(p.g),
                beta=np.ascontiguousarray(p.beta),
                qk_row=p.nk * HEAD_DIM, v_row=p.nv * HEAD_DIM, gb_row=p.nv)


def pack_conv(p):
    """One bf16 buffer ``[N][conv_dim]`` holding q (column 0), k (column
    nk*128) and v (column 2*nk*128), ``conv_dim = 2*nk*128 + nv*128``; one f32
    buffer ``[N][2*nv]`` holding g (column 0) and beta (column nv) -- the
    packed conv layout of the page's launcher (``qk_stride = v_stride =
    conv_dim``, ``gb_stride = 2*nv``)."""
    N = p.n_tokens
    qk = p.nk * HEAD_DIM
    conv_dim = 2 * qk + p.nv * HEAD_DIM
    conv = np.empty((N, conv_dim), dtype=np.uint16)
    conv[:, :qk] = p.q.reshape(N, qk)
    conv[:, qk:2 * qk] = p.k.reshape(N, qk)
    conv[:, 2 * qk:] = p.v.reshape(N, p.nv * HEAD_DIM)
    gb = np.empty((N, 2 * p.nv), dtype=np.float32)
    gb[:, :p.nv] = p.g
    gb[:, p.nv:] = p.beta
    return dict(conv=conv, gb=gb, q_off=0, k_off=qk, v_off=2 * qk, g_off=0, beta_off=p.nv,
                qk_row=conv_dim, v_row=conv_dim, gb_row=2 * p.nv)
