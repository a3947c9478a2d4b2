// Stage 1: chunk_cumsum_recompute_wu.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 1: per chunk and v-head, the chunk-local cumulative log-gate gc and the
// WY/UT solves (I+L) U = beta V, (I+L) W = beta exp(gc) K, with L sharing the
// key Gram matrix's buffer (comment above smem_wu).  For the chunk's n <= 64
// tokens (rows past the sequence end are zero):
//   G_r    = sum_{j<=r} g_j
//   L[r,s] = beta_r exp(G_r - G_s) (k_r . k_s)        (s < r, else 0)
//   T'     = (I + L)^-1 diag(beta)                     (the UT transform)
// so that U = T' V and W = T' diag(exp(G)) K.  This stage emits T' itself
// (10 KB per chunk-head) instead of W and U (64 KB in float32): the spine forms
// uc = U - W h = T' (V - diag(exp(G)) K h) on the fly from T', K and V.
//
// One wave per (chunk, v-head):
//   * lane t scans g; emits gc, exp(G_t) and exp(G_{n-1} - G_t);
//   * the lower 10 tiles of K K^T on bf16 MFMA (K is exact in bf16) -> L (f32,
//     LDS, its three lower 32x32 blocks only: 12.8 KB, so that 12 workgroups
//     fit a CU);
//   * the two diagonal 32x32 blocks of T = (I+L)^-1 by f32 forward
//     substitution, one lane per column (32 rows, <= 496 FMAs per lane);
//   * the off-diagonal block T21 = -T22 (L21 T11) on MFMA, every operand split
//     into bf16 hi + lo (three products each, ~2^-17 relative error);
//   * T' = T diag(beta), split hi/lo, stored in the A-operand fragment order
//     the spine reads (hi and lo: the 6 nonzero fragments x 64 lanes x 16
//     bytes, of which the two diagonal fragments keep only the first 8 bytes
//     per lane, their other half being the zero block above the diagonal).
#include "gdn_device.h"

namespace gdn {

constexpr int kBP = 32; // pitch (floats) of the 32x32 L / T blocks (12.8 KB of LDS: 12 workgroups per CU)

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
  const int q4 = lane >> 4, r16 = lane & 15;

  // The three 32x32 blocks of the lower-triangular L, overwritten in place by
  // the blocks of T = (I + L)^-1: B[0] = L11 / T11 (rows 0..31, columns 0..31),
  // B[1] = L21 / T21 (rows 32..63, columns 0..31), B[2] = L22 / T22 (rows
  // 32..63, columns 32..63).  T12 = 0 is never stored.
  __shared__ __align__(16) float Bk[3][32 * kBP];
  __shared__ float Gs[kChunk], Bs[kChunk];
  // element (r, s), r >= s / 32 * 32, of L / T
  auto at = [&](int r, int sc) -> float * {
    return &Bk[r < 32 ? 0 : (sc < 32 ? 1 : 2)][(r & 31) * kBP + (sc & 31)];
  };

  // ---- K rows in the contiguous k order: kf[m][kb] = K[16m + r16][32kb + 8q .. +7]
  const uint16_t *kbase = p.k + row0 * p.qk_row + int64_t(kh) * kDim;
  bf16x8 kf[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + r16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kf[m][kb] = (t < n) ? load16_bf16x8(kbase + int64_t(t) * p.qk_row + 32 * kb + 8 * q4) : zero8();
  }

  // ---- gate: inclusive prefix sum over the chunk (g = 0 past the end) -----
  {
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
    const float Gn = __shfl(G, n - 1, 64);
    Gs[lane] = G * 1.4426950408889634f; // log2(e) G, for exp2 below
    Bs[lane] = bv;
    p.gc[slot * kChunk + lane] = G;
    p.dec[slot * 2 * kChunk + lane] = expf(G);
    p.dec[slot * 2 * kChunk + kChunk + lane] = expf(Gn - G);
  }

  // ---- L = strict_lower(diag(beta) (D * K K^T)) ---------------------------
#pragma unroll
  for (int mr = 0; mr < 4; ++mr)
#pragma unroll
    for (int ms = 0; ms <= mr; ++ms) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(kf[mr][kb], kf[ms][kb], acc);
      const int sc = 16 * ms + r16; // C tile: column s, rows r
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * mr + 4 * q4 + ii;
        *at(r, sc) = (sc < r) ? Bs[r] * __builtin_amdgcn_exp2f(Gs[r] - Gs[sc]) * acc[ii] : 0.f;
      }
    }

  // ---- diagonal blocks: T_bb = (I + L_bb)^-1, lane j owns column j of block
  // b = j / 32:  T[r][j] = delta_rj - sum_{s<r} L[r][s] T[s][j] -------------
  {
    const int b = lane >> 5, jj = lane & 31;
    float *blk = Bk[b ? 2 : 0];
    float t[32];
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      float a0 = (rr == jj) ? 1.f : 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      const float *Lr = blk + rr * kBP;
#pragma unroll
      for (int s4 = 0; s4 < rr / 4; ++s4) {
        const f32x4 lv = *reinterpret_cast<const f32x4 *>(Lr + 4 * s4);
        a0 -= lv[0] * t[4 * s4 + 0];
        a1 -= lv[1] * t[4 * s4 + 1];
        a2 -= lv[2] * t[4 * s4 + 2];
        a3 -= lv[3] * t[4 * s4 + 3];
      }
#pragma unroll
      for (int s1 = 4 * (rr / 4); s1 < rr; ++s1) a0 -= Lr[s1] * t[s1];
      t[rr] = (a0 + a1) + (a2 + a3);
    }
    // T11 and T22 in place of L11 and L22 (their reads are done)
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) blk[rr * kBP + jj] = t[rr];
  }

  // ---- T21 = -T22 (L21 T11): rows 32..63, columns 0..31 -------------------
  {
    // Pm = L21 T11, contiguous k order over s in [0, 32); T11's columns are
    // read straight from its rows (16 lanes read 16 consecutive floats)
    f32x4 Pm[2][2];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp) {
      const float *ar = Bk[1] + (16 * mp + r16) * kBP + 8 * q4;
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(ar);
      const f32x4 a1 = *reinterpret_cast<const f32x4 *>(ar + 4);
      const float xa[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      bf16x8 ah, al;
      split8(xa, ah, al);
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = Bk[0][(8 * q4 + e) * kBP + 16 * np + r16];
        bf16x8 bh, bl;
        split8(xb, bh, bl);
        f32x4 acc = mfma(ah, bh, zero4());
        acc = mfma(ah, bl, acc);
        Pm[mp][np] = mfma(al, bh, acc);
      }
    }
    // T21 = -T22 Pm; Pm's C tiles are the B operand in chain order over s'
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int np = 0; np < 2; ++np) chain_split(Pm[0][np], Pm[1][np], ph[np], pl[np]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float *ar = Bk[2] + (16 * mt + r16) * kBP + 4 * q4;
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(ar);
      const f32x4 a1 = *reinterpret_cast<const f32x4 *>(ar + 16);
      const float xa[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      bf16x8 ah, al;
      split8(xa, ah, al);
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        f32x4 acc = mfma(ah, ph[np], zero4());
        acc = mfma(ah, pl[np], acc);
        acc = mfma(al, ph[np], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Bk[1][(16 * mt + 4 * q4 + ii) * kBP + 16 * np + r16] = -acc[ii];
      }
    }
  }

  // ---- T' = T diag(beta) in the spine's A-operand order: fragment (mt, kb)
  // holds rows t = 16mt + r16, columns s = 32kb + {4q..4q+3, 16+4q..16+4q+3};
  // only the six with mt >= 2kb are stored (T' is lower triangular): the hi
  // parts, then the lo parts, 16 bytes per lane ------------------------------
  char *dst = reinterpret_cast<char *>(p.tp + slot * (kTpBytes / 2));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (2 * kb > mt) continue;
      const int t = 16 * mt + r16;
      const int s0 = 32 * kb + 4 * q4, s1 = s0 + 16;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(at(t, s0));
      const f32x4 b = *reinterpret_cast<const f32x4 *>(at(t, s1));
      const float x[8] = {a[0] * Bs[s0], a[1] * Bs[s0 + 1], a[2] * Bs[s0 + 2], a[3] * Bs[s0 + 3],
                          b[0] * Bs[s1], b[1] * Bs[s1 + 1], b[2] * Bs[s1 + 2], b[3] * Bs[s1 + 3]};
      bf16x8 hi, lo;
      split8(x, hi, lo);
      const int f = tri_frag(mt, kb);
      const u32x4 h4 = __builtin_bit_cast(u32x4, hi), l4 = __builtin_bit_cast(u32x4, lo);
      if (tp_half(f)) { // columns 32kb + 16.. are above the diagonal: zero
        *reinterpret_cast<u32x2 *>(dst + tp_offset(f) + 8 * lane) = u32x2{h4[0], h4[1]};
        *reinterpret_cast<u32x2 *>(dst + kTpPartBytes + tp_offset(f) + 8 * lane) = u32x2{l4[0], l4[1]};
      } else {
        *reinterpret_cast<u32x4 *>(dst + tp_offset(f) + 16 * lane) = h4;
        *reinterpret_cast<u32x4 *>(dst + kTpPartBytes + tp_offset(f) + 16 * lane) = l4;
      }
    }
}

hipError_t launch_stage1(const Params &p, hipStream_t stream) {
  dim3 grid(unsigned(((p.max_chunks + 7) / 8) * 8 * p.nv), p.B);
  hipLaunchKernelGGL(chunk_cumsum_recompute_wu, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
