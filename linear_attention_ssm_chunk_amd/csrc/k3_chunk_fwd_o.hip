// Stage 3: chunk_fwd_o, the per-chunk output.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 3: O = Q~ S_c + tril(decay * Q~ K^T) uc, bf16 out.  Read so that it
// equals the recurrence's o_t = S_t q_t (the state after token t):
//   O[t] = exp(G_t) q_t h_c + sum_{s<=t} exp(G_t - G_s) (q_t . k_s) uc[s]
// with h_c the chunk's entry state and uc = U - W h_c from stage 2.
// One 256-thread workgroup per (chunk, v-head); wave w produces value
// columns [32w, 32w+32) for all 64 tokens.  No LDS:
//   * P^T = K Q^T (16x16 tiles, s <= t) lands in C layout with column t and
//     rows s, which in chain order is the A operand of P uc -- mask and decay
//     are applied in registers;
//   * the entry state (stored [dk][dv]) becomes the B operand of Q h_c through
//     an identity product;
//   * O is rounded to bf16 and turned by an identity product so that each lane
//     stores 4 consecutive dv of one token (8-byte stores).
#include "gdn_device.h"

namespace gdn {

__global__ __launch_bounds__(kThreads) void chunk_fwd_o(Params p) {
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Seq s = seq_of(p, i);
  if (!s.ok || c >= s.nchunks) return;
  const int n = min(kChunk, s.len - c * kChunk);
  const int64_t slot = slot_of(p, s, h, c);
  const int kh = (h * p.nk) / p.nv;
  const int64_t row0 = s.tok0 + int64_t(c) * kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int dvw = 32 * wave;
  const float *gcp = p.gc + slot * kChunk;

  // q, k rows 16m + r16 in chain order over dk (zero past the sequence end)
  const uint16_t *qb = p.q + row0 * p.qk_row + int64_t(kh) * kDim;
  const uint16_t *kb_ = p.k + row0 * p.qk_row + int64_t(kh) * kDim;
  bf16x8 qf[4][4], kf[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + r16;
    const bool ok = t < n;
    const uint16_t *qr = qb + int64_t(t) * p.qk_row + 4 * q4;
    const uint16_t *kr = kb_ + int64_t(t) * p.qk_row + 4 * q4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qf[m][kb] = ok ? join8(load8(qr + 32 * kb), load8(qr + 32 * kb + 16)) : zero8();
      kf[m][kb] = ok ? join8(load8(kr + 32 * kb), load8(kr + 32 * kb + 16)) : zero8();
    }
  }

  // decayed, causally masked scores as A operands: aq[mt][kb] covers tokens
  // t = 16mt + r16 and s in [32kb, 32kb+32)
  bf16x8 aq[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = 16 * mt + r16;
    const float Gt = gcp[t];
    f32x4 P[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      P[ms] = zero4();
      if (ms <= mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mfma(kf[ms][kb], qf[mt][kb], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int si = 16 * ms + 4 * q4 + ii;
          P[ms][ii] = (si <= t) ? expf(Gt - gcp[si]) * acc[ii] : 0.f;
        }
      }
    }
    aq[mt][0] = chain_frag(P[0], P[1]);
    aq[mt][1] = chain_frag(P[2], P[3]);
  }

  // entry state columns [dvw, dvw+32) as B operands (k = dk, chain order)
  bf16x8 sB[4][2];
  {
    const bf16x8 I0 = ident_contig(lane, 0), I1 = ident_contig(lane, 1);
    const uint16_t *sp = p.s_entry + slot * (kDim * kDim) + dvw + 8 * q4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 s0 = load16_bf16x8(sp + (32 * kb + r16) * kDim);
      const bf16x8 s1 = load16_bf16x8(sp + (32 * kb + 16 + r16) * kDim);
      sB[kb][0] = chain_frag(mfma(s0, I0, zero4()), mfma(s1, I0, zero4()));
      sB[kb][1] = chain_frag(mfma(s0, I1, zero4()), mfma(s1, I1, zero4()));
    }
  }

  // corrected values uc (stored [dv][token]) as B operands (k = token, chain)
  bf16x8 dB[2][2];
  {
    const uint16_t *up = p.uc + slot * (kDim * kChunk) + 4 * q4;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint16_t *ur = up + (dvw + 16 * b + r16) * kChunk;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dB[kb][b] = join8(load8(ur + 32 * kb), load8(ur + 32 * kb + 16));
    }
  }

  // O tiles: C layout column dv = dvw + 16b + r16, rows t = 16mt + 4q .. +3
  f32x4 O[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float eg[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) eg[ii] = expf(gcp[16 * mt + 4 * q4 + ii]);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(qf[mt][kb], sB[kb][b], acc);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) acc[ii] *= eg[ii];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (2 * kb <= mt) acc = mfma(aq[mt][kb], dB[kb][b], acc);
      O[mt][b] = acc;
    }
  }

  // bf16, transpose by identity, store 4 dv of one token per lane
  const bf16x8 C0 = ident_chain(lane, 0), C1 = ident_chain(lane, 1);
  const int64_t orow = int64_t(p.nv) * kDim;
  uint16_t *ob = p.out + row0 * orow + int64_t(h) * kDim + dvw + 4 * q4;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 oa = chain_frag(O[2 * kk][b], O[2 * kk + 1][b]);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4 d = mfma(oa, half ? C1 : C0, zero4());
        const int t = 32 * kk + 16 * half + r16;
        if (t < n) *reinterpret_cast<u32x2 *>(ob + int64_t(t) * orow + 16 * b) = pack4_bf16(d[0], d[1], d[2], d[3]);
      }
    }
}

hipError_t launch_stage3(const Params &p, hipStream_t stream) {
  dim3 grid(p.max_chunks, p.nv, p.B);
  hipLaunchKernelGGL(chunk_fwd_o, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
