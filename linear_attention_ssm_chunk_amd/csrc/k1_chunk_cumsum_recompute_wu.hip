// Stage 1: chunk_cumsum_recompute_wu.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 1: per chunk and v-head, the chunk-local cumulative log-gate gc and the
// solves (I+L) U = beta V, (I+L) W = beta exp(gc) K, with L sharing the key Gram
// matrix's buffer (comment above smem_wu).  Here, for the chunk's n <= 64
// tokens (rows past the sequence end are zero):
//   G_r    = sum_{j<=r} g_j
//   L[r,s] = beta_r exp(G_r - G_s) (k_r . k_s)        (s < r, else 0)
//   T      = (I + L)^-1                               (unit lower triangular)
//   U      = T diag(beta) V,   W = T diag(beta exp(G)) K
// Work split of one 256-thread workgroup:
//   wave 0      prefix sum of g (one lane per token)
//   wave w      Gram tiles (w, 0..w) on bf16 MFMA -> L in LDS (f32)
//   wave 0      T by forward substitution, one lane per column, f32
//   wave w      W^T, U^T rows d in [32w, 32w+32): bf16 MFMA with K, V exact and
//               T split hi+lo (two products), f32 out.
// K and V are turned into k = token operands by identity products in
// registers (see gdn_device.h), so the only LDS tile is L / T' (17 KB).
#include "gdn_device.h"

namespace gdn {

constexpr int kLP = 68; // row pitch (floats) of the L / T' tile

__global__ __launch_bounds__(kThreads) void chunk_cumsum_recompute_wu(Params p) {
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Seq s = seq_of(p, i);
  if (!s.ok || c >= s.nchunks) return;
  const int n = min(kChunk, s.len - c * kChunk);
  const int64_t slot = slot_of(p, s, h, c);
  const int kh = (h * p.nk) / p.nv;
  const int64_t row0 = s.tok0 + int64_t(c) * kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;

  __shared__ __align__(16) float Ls[kChunk * kLP];
  __shared__ float Gs[kChunk], Bs[kChunk], Es[kChunk];

  // --- gc: inclusive prefix sum of g over the chunk (g = 0 past the end, so
  // padded rows repeat the last value) ---------------------------------------
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (lane < n) {
      const int64_t off = (row0 + lane) * p.gb_row + h;
      gv = p.g[off];
      bv = p.beta[off];
    }
    float G = gv;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(G, d, 64);
      if (lane >= d) G += o;
    }
    Gs[lane] = G;
    Bs[lane] = bv;
    Es[lane] = expf(G);
    p.gc[slot * kChunk + lane] = G;
  }

  // --- operands straight from HBM (16-byte loads, rows past the end = 0) ----
  const uint16_t *kbase = p.k + row0 * p.qk_row + int64_t(kh) * kDim;
  const uint16_t *vbase = p.v + row0 * p.v_row + int64_t(h) * kDim;
  // kf[m][kb] = K[16m + r16][32kb + 8q .. +7]: B operands of the Gram
  bf16x8 kf[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + r16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kf[m][kb] = (t < n) ? load16_bf16x8(kbase + int64_t(t) * p.qk_row + 32 * kb + 8 * q4) : zero8();
  }
  // ka[kb]: A operands of this wave's Gram row tile (rows 16*wave + r16)
  bf16x8 ka[4];
  {
    const int t = 16 * wave + r16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      ka[kb] = (t < n) ? load16_bf16x8(kbase + int64_t(t) * p.qk_row + 32 * kb + 8 * q4) : zero8();
  }
  // this wave's 32 columns of K and V, natural orientation (for transposing)
  bf16x8 kc[4], vc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + r16;
    const bool ok = t < n;
    kc[m] = ok ? load16_bf16x8(kbase + int64_t(t) * p.qk_row + 32 * wave + 8 * q4) : zero8();
    vc[m] = ok ? load16_bf16x8(vbase + int64_t(t) * p.v_row + 32 * wave + 8 * q4) : zero8();
  }

  __syncthreads(); // Gs, Bs, Es

  // --- Gram row tile `wave`, column tiles 0..wave -> L --------------------
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (ns <= wave) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(ka[kb], kf[ns][kb], acc);
      const int sc = 16 * ns + r16; // C: column s, rows r
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * wave + 4 * q4 + ii;
        Ls[r * kLP + sc] = (sc < r) ? Bs[r] * expf(Gs[r] - Gs[sc]) * acc[ii] : 0.f;
      }
    }
  }

  // --- K, V columns [32w, 32w+32) transposed in registers: kA[kb][b] is the
  // A operand (rows d = 32w + 16b + r16, k = tokens, chain order) ------------
  bf16x8 kA[2][2], vA[2][2];
  {
    const bf16x8 I0 = ident_contig(lane, 0), I1 = ident_contig(lane, 1);
    f32x4 kt[4][2], vt[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kt[m][0] = mfma(kc[m], I0, zero4());
      kt[m][1] = mfma(kc[m], I1, zero4());
      vt[m][0] = mfma(vc[m], I0, zero4());
      vt[m][1] = mfma(vc[m], I1, zero4());
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        kA[kb][b] = chain_frag(kt[2 * kb][b], kt[2 * kb + 1][b]);
        vA[kb][b] = chain_frag(vt[2 * kb][b], vt[2 * kb + 1][b]);
      }
  }

  __syncthreads(); // L complete

  // --- T = (I + L)^-1 by forward substitution; lane j owns column j:
  //     T[r][j] = delta_rj - sum_{s<r} L[r][s] T[s][j]
  // then T' = T diag(beta) overwrites L in place (all reads of L are done). --
  if (wave == 0) {
    const int j = lane;
    float t[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
      float a0 = (r == j) ? 1.f : 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      const float *Lr = Ls + r * kLP;
#pragma unroll
      for (int s4 = 0; s4 < r / 4; ++s4) {
        const f32x4 lv = *reinterpret_cast<const f32x4 *>(Lr + 4 * s4);
        a0 -= lv[0] * t[4 * s4 + 0];
        a1 -= lv[1] * t[4 * s4 + 1];
        a2 -= lv[2] * t[4 * s4 + 2];
        a3 -= lv[3] * t[4 * s4 + 3];
      }
#pragma unroll
      for (int s1 = 4 * (r / 4); s1 < r; ++s1) a0 -= Lr[s1] * t[s1];
      t[r] = (a0 + a1) + (a2 + a3);
    }
    const float bj = Bs[j];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) Ls[r * kLP + j] = t[r] * bj;
  }

  __syncthreads(); // T' ready

  // --- W^T[d][t] = sum_s K^T[d][s] T''[t][s],  T'' = T' diag(exp(G));
  //     U^T[d][t] = sum_s V^T[d][s] T'[t][s].
  // C tile: column t = 16nt + r16, rows d = 32w + 16b + 4q .. +3 -> one float4
  // store into row-major W[t][d]. ------------------------------------------
  float *wout = p.w + slot * (kChunk * kDim);
  float *uout = p.u + slot * (kChunk * kDim);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = 16 * nt + r16;
    bf16x8 twh[2], twl[2], tuh[2], tul[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(Ls + t * kLP + 32 * kb + 4 * q4);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(Ls + t * kLP + 32 * kb + 16 + 4 * q4);
      float xu[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      float xw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sidx = 32 * kb + ((e < 4) ? 4 * q4 + e : 16 + 4 * q4 + (e - 4));
        xw[e] = xu[e] * Es[sidx];
      }
      split8(xu, tuh[kb], tul[kb]);
      split8(xw, twh[kb], twl[kb]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 aw = zero4(), au = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        aw = mfma(kA[kb][b], twh[kb], aw);
        aw = mfma(kA[kb][b], twl[kb], aw);
        au = mfma(vA[kb][b], tuh[kb], au);
        au = mfma(vA[kb][b], tul[kb], au);
      }
      const int d = 32 * wave + 16 * b + 4 * q4;
      *reinterpret_cast<f32x4 *>(wout + t * kDim + d) = aw;
      *reinterpret_cast<f32x4 *>(uout + t * kDim + d) = au;
    }
  }
}

hipError_t launch_stage1(const Params &p, hipStream_t stream) {
  dim3 grid(p.max_chunks, p.nv, p.B);
  hipLaunchKernelGGL(chunk_cumsum_recompute_wu, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
