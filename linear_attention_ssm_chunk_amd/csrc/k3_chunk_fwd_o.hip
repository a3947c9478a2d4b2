// Stage 3: chunk_fwd_o, the per-chunk output.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 3: O = Q~ S_c + tril(decay * Q~ K^T) uc, bf16 out.  Read so that it
// equals the recurrence's o_t = S_t q_t (the state after token t):
//   O[t] = exp(G_t) S_c q_t + sum_{s<=t} exp(G_t - G_s) (q_t . k_s) uc[s]
// with S_c the chunk's entry state (stored [dv][dk]) and uc from stage 2.
//
// One 256-thread workgroup per (chunk, v-head):
//   1. Q and K tiles (64 x 128 bf16) are loaded once, row-coalesced, into LDS.
//   2. Wave w computes the scores of token tile w, P^T = K Q^T for s-tiles
//      0..w, applies the causal mask and exp(G_t - G_s) in registers, and
//      writes the bf16 scores to LDS (one pass, no redundancy).
//   3. Wave w then owns value columns [32w, 32w+32) for all 64 tokens:
//      exp(G) * (Q S_c^T) + A uc on bf16 MFMA, with S_c and uc read straight
//      from HBM in the operand order (16-byte loads, no transposes).
//   4. O is rounded to bf16, turned by an identity product so each lane holds
//      4 consecutive columns of a token, staged in LDS, and stored as whole
//      256-byte rows.
#include "gdn_device.h"

namespace gdn {

constexpr int kQP = 136; // Q / K / O tile pitch (bf16): 272-byte rows
constexpr int kAP = 72;  // score tile pitch (bf16): 144-byte rows

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

  __shared__ __align__(16) uint16_t Qs[kChunk * kQP]; // later: O staging
  __shared__ __align__(16) uint16_t Ks[kChunk * kQP];
  __shared__ __align__(16) uint16_t As[kChunk * kAP];
  __shared__ float G2[kChunk], EG[kChunk];

  // ---- operands this wave reads from HBM, issued first ---------------------
  // entry state columns dv = dvw + 16b + r16, contiguous dk (B operand of Q S^T)
  bf16x8 sB[4][2];
  {
    const uint16_t *sp = p.s_entry + slot * (kDim * kDim) + 8 * q4;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sB[kb][b] = load16_bf16x8(sp + (dvw + 16 * b + r16) * kDim + 32 * kb);
  }
  // uc columns dv, contiguous tokens (B operand of A uc)
  bf16x8 uB[2][2];
  {
    const uint16_t *up = p.uc + slot * (kDim * kChunk) + 8 * q4;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) uB[kb][b] = load16_bf16x8(up + (dvw + 16 * b + r16) * kChunk + 32 * kb);
  }

  // ---- Q, K tiles -> LDS (rows past the end are 0) -------------------------
  {
    const int cc = tid & 15, rr = tid >> 4;
    const uint16_t *qsrc = p.q + row0 * p.qk_row + int64_t(kh) * kDim + 8 * cc;
    const uint16_t *ksrc = p.k + row0 * p.qk_row + int64_t(kh) * kDim + 8 * cc;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int t = rr + 16 * jj;
      const bool ok = t < n;
      const u32x4 qv = ok ? *reinterpret_cast<const u32x4 *>(qsrc + int64_t(t) * p.qk_row) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 kv = ok ? *reinterpret_cast<const u32x4 *>(ksrc + int64_t(t) * p.qk_row) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(Qs + t * kQP + 8 * cc) = qv;
      *reinterpret_cast<u32x4 *>(Ks + t * kQP + 8 * cc) = kv;
    }
    if (tid < kChunk) {
      G2[tid] = p.gc[slot * kChunk + tid] * 1.4426950408889634f; // log2(e)
      EG[tid] = p.dec[slot * 2 * kChunk + tid];                  // exp(G_t)
    }
  }
  __syncthreads();

  // ---- scores of token tile w: A[t][s] = exp(G_t - G_s) q_t.k_s, s <= t ----
  {
    const int t = 16 * wave + r16;
    bf16x8 qb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = *reinterpret_cast<const bf16x8 *>(Qs + t * kQP + 32 * kb + 8 * q4);
    const float gt = G2[t];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      u32x2 packed = {0u, 0u};
      if (ms <= wave) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(Ks + (16 * ms + r16) * kQP + 32 * kb + 8 * q4);
          acc = mfma(ka, qb[kb], acc);
        }
        // C tile: column t, rows s = 16ms + 4q .. +3
        float v4[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int si = 16 * ms + 4 * q4 + ii;
          v4[ii] = (si <= t) ? __builtin_amdgcn_exp2f(gt - G2[si]) * acc[ii] : 0.f;
        }
        packed = pack4_bf16(v4[0], v4[1], v4[2], v4[3]);
      }
      *reinterpret_cast<u32x2 *>(As + t * kAP + 16 * ms + 4 * q4) = packed;
    }
  }
  __syncthreads();

  // ---- O columns [dvw, dvw+32): C tile (mt, b): column dv, rows t -----------
  f32x4 O[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = 16 * mt + r16;
    bf16x8 qa[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qa[kb] = *reinterpret_cast<const bf16x8 *>(Qs + t * kQP + 32 * kb + 8 * q4);
    bf16x8 aa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) aa[kb] = *reinterpret_cast<const bf16x8 *>(As + t * kAP + 32 * kb + 8 * q4);
    float eg[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) eg[ii] = EG[16 * mt + 4 * q4 + ii];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(qa[kb], sB[kb][b], acc);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) acc[ii] *= eg[ii];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (2 * kb <= mt) acc = mfma(aa[kb], uB[kb][b], acc);
      O[mt][b] = acc;
    }
  }
  __syncthreads(); // every wave is done reading Qs: reuse it for O

  // ---- bf16, identity transpose (lane: 4 consecutive dv of one token), LDS --
  uint16_t *Os = Qs;
  {
    const bf16x8 C0 = ident_chain(lane, 0), C1 = ident_chain(lane, 1);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 oa = chain_frag(O[2 * kk][b], O[2 * kk + 1][b]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 d = mfma(oa, half ? C1 : C0, zero4());
          const int t = 32 * kk + 16 * half + r16;
          *reinterpret_cast<u32x2 *>(Os + t * kQP + dvw + 16 * b + 4 * q4) = pack4_bf16(d[0], d[1], d[2], d[3]);
        }
      }
  }
  __syncthreads();

  // ---- whole-row stores: out[row0 + t][h][0..127] ---------------------------
  {
    const int cc = tid & 15, rr = tid >> 4;
    const int64_t orow = int64_t(p.nv) * kDim;
    uint16_t *ob = p.out + row0 * orow + int64_t(h) * kDim + 8 * cc;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int t = rr + 16 * jj;
      if (t < n) *reinterpret_cast<u32x4 *>(ob + int64_t(t) * orow) = *reinterpret_cast<const u32x4 *>(Os + t * kQP + 8 * cc);
    }
  }
}

hipError_t launch_stage3(const Params &p, hipStream_t stream) {
  dim3 grid(p.max_chunks, p.nv, p.B);
  hipLaunchKernelGGL(chunk_fwd_o, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
