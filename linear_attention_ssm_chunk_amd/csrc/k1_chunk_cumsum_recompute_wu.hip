// Stage 1: chunk_cumsum_recompute_wu.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 1: per chunk and v-head, the chunk-local cumulative log-gate gc and the
// WY/UT solve (gdn_ut_solve.h), written to the scratch: gc and
// T' = (I+L)^-1 diag(beta) (10 KB per chunk-head as a bf16 hi + lo pair, so
// that U = T' V and W = T' diag(exp(G)) K) -- not W and U (64 KB in float32).  With q/k
// normalisation it also writes the row scales 1/|k_t| and 1/|q_t| of the
// chunk, which the spine folds into its decays.
//
// One wave per (chunk, v-head).  T' leaves as bf16 hi, then bf16 lo, each in
// the spine's A-operand fragment order: the 6 nonzero fragments x 64 lanes x
// 16 bytes, of which the two diagonal fragments keep only the first 8 bytes
// per lane (their other half is the zero block above the diagonal).
#include "gdn_ut_solve.h"

namespace gdn {

template <bool kNorm>
__global__ __launch_bounds__(64) void chunk_cumsum_recompute_wu(Params p) {
  // Workgroup order: all nv heads of one chunk get ids 8 apart, so that on a
  // round-robin XCD dispatch they run close together on one XCD and share its
  // L2 -- the chunk's K rows (each read by the r = nv/nk v-heads of a k-head,
  // which come one after another) and its g / beta rows (one row per token
  // holds every head's value).
  const int xcd = blockIdx.x & 7, round = blockIdx.x >> 3;
  const int c = (round / p.nv) * 8 + xcd, h = round % p.nv, i = blockIdx.y;
  const Seq s = seq_of(p, i);
  if (c >= p.max_chunks || !s.ok || c >= s.nchunks) return;
  const int n = min(kChunk, s.len - c * kChunk);
  const int64_t slot = slot_of(p, s, h, c);
  const int kh = (h * p.nk) / p.nv;
  const int64_t row0 = s.tok0 + int64_t(c) * kChunk;
  const int lane = threadIdx.x;

  __shared__ UtWork work;
  bf16x8 kf[4][4];
  load_k_frags(kf, p.k + row0 * p.qk_row + int64_t(kh) * kDim, p.qk_row, n, lane);
  float gv = 0.f, bv = 0.f;
  if (lane < n) {
    const int64_t off = (row0 + lane) * p.gb_row + h;
    gv = p.g[off];
    bv = p.beta[off];
  }
  float sk = 1.f;
  if (kNorm) {
    // both row scales are formed here, where a row's pieces sit in four lanes
    // (the spine's loaders read whole rows, 16 lanes each, and would need a
    // longer reduction on waves that share a SIMD with the state's products)
    bf16x8 qf[4][4];
    load_k_frags(qf, p.q + row0 * p.qk_row + int64_t(kh) * kDim, p.qk_row, n, lane);
    const float sq = inv_row_norm(qf, lane);
    sk = inv_row_norm(kf, lane);
    p.nrm[slot * 2 * kChunk + lane] = sk;
    p.nrm[slot * 2 * kChunk + kChunk + lane] = sq;
  }
  u32x4 tx[2 * kTpFrags];
  float G, Gn;
  ut_solve<kNorm>(kf, gv, bv, sk, n, work, lane, tx, G, Gn);

  p.gc[slot * kChunk + lane] = G;
  char *dst = reinterpret_cast<char *>(p.tp) + slot * kTpBytes;
#pragma unroll
  for (int part = 0; part < 2; ++part)
#pragma unroll
    for (int f = 0; f < kTpFrags; ++f) {
      const u32x4 &x = tx[part * kTpFrags + f];
      char *d = dst + part * kTpHalfBytes + tp_offset(f);
      if (tp_half(f)) // the second half lies above the diagonal: zero, not stored
        *reinterpret_cast<u32x2 *>(d + 8 * lane) = u32x2{x[0], x[1]};
      else
        *reinterpret_cast<u32x4 *>(d + 16 * lane) = x;
    }
}

hipError_t launch_stage1(const Params &p, hipStream_t stream) {
  dim3 grid(unsigned(((p.max_chunks + 7) / 8) * 8 * p.nv), p.B);
  if (p.opts & kOptNorm)
    hipLaunchKernelGGL(chunk_cumsum_recompute_wu<true>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(chunk_cumsum_recompute_wu<false>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
