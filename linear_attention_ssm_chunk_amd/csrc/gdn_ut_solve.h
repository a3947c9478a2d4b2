// gdn_ut_solve.h -- the per-chunk gate scan and UT solve, one wave per
// (chunk, v-head), shared by the stage that emits its results
// (chunk_cumsum_recompute_wu) and the spine that forms them on the fly.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 1: the chunk-local cumulative log-gate gc and the WY/UT solves
// (I+L) U = beta V, (I+L) W = beta exp(gc) K, with L sharing the key Gram
// matrix's buffer (comment above smem_wu).  For the chunk's n <= 64 tokens
// (lanes and rows past the sequence end carry g = beta = 0):
//   G_r    = sum_{j<=r} g_j
//   L[r,s] = beta_r exp(G_r - G_s) (k_r . k_s)        (s < r, else 0)
//   T'     = (I + L)^-1 diag(beta)                     (the UT transform)
// so that U = T' V and W = T' diag(exp(G)) K.
// T = (I+L)^-1 by blocks: for a unit lower-triangular [[A, 0], [C, D]], the
// inverse is [[A^-1, 0], [-D^-1 C A^-1, D^-1]].
//   * lane t scans g;
//   * the lower 10 16x16 tiles of K K^T on bf16 MFMA (K is exact in bf16) ->
//     L (f32, LDS, one row-major tile each);
//   * the four diagonal 16x16 tiles of T by f32 forward substitution, one lane
//     per column of each (<= 120 FMAs per lane);
//   * the off-diagonal tiles of the two diagonal 32x32 blocks, then the lower
//     left 32x32 block, by the formula above on MFMA, every operand split
//     into bf16 hi + lo (three products each, ~2^-17 relative error);
//   * T' = T diag(beta), rounded to float16 (11 significant bits: the spine
//     splits each value exactly into bf16 hi + lo), in the A-operand fragment
//     order of the spine: fragment f = tri_frag(mt, kb) (mt >= 2kb) holds, in
//     lane 16q + r, row t = 16mt + r, columns s = 32kb + 4q + e and
//     32kb + 16 + 4q + e (e = 0..3).  In the diagonal fragments (mt = 2kb)
//     the second four lie above the diagonal and are 0.
#pragma once

#include "gdn_device.h"

namespace gdn {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Tiles of L / T: tile (mr, ms), ms <= mr, holds rows 16mr.., columns 16ms..
// row-major with a pitch of kTP floats; tiles lie kTileF floats apart.  The
// pitch puts the 4 rows x 16 columns a wave writes from a C fragment in 64
// distinct banks; the extra 4 floats per tile put the four diagonal tiles,
// which the substitution reads at once, in different banks.
constexpr int kTP = 20;
constexpr int kTileF = 16 * kTP + 4;
__host__ __device__ constexpr int tri_tile(int mr, int ms) { return mr * (mr + 1) / 2 + ms; }

// LDS workspace of one solving wave (13.2 KB).
struct __align__(16) UtWork {
  float L[10 * kTileF];
  float Gs[kChunk]; // log2(e) G_t, for exp2
  float Bs[kChunk]; // beta_t
};

// hi = bf16(x), lo = bf16(x - hi) for pairs of floats; x - hi is exact in
// float32 and comes from one bf16 dot product, (hi0, hi1) . (-1, 0) + x0, with
// the constant pairs in registers m0, m1 (an inline constant would be read as
// the float32 -1.0).
struct SplitK {
  uint32_t m0, m1;
  __device__ __forceinline__ SplitK() : m0(0x0000BF80u), m1(0xBF800000u) {
    asm volatile("" : "+v"(m0));
    asm volatile("" : "+v"(m1));
  }
  __device__ __forceinline__ void pair(float a, float b, uint32_t &hi, uint32_t &lo) const {
    hi = cvt_pk(a, b);
    const bf16x2 h2 = __builtin_bit_cast(bf16x2, hi);
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(h2, __builtin_bit_cast(bf16x2, m0), a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(h2, __builtin_bit_cast(bf16x2, m1), b, false);
    lo = cvt_pk(ra, rb);
  }
  __device__ __forceinline__ void four(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) const {
    uint32_t h0, h1, l0, l1;
    pair(x[0], x[1], h0, l0);
    pair(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
  }
  __device__ __forceinline__ void eight(const f32x4 &x, const f32x4 &y, bf16x8 &hi, bf16x8 &lo) const {
    uint32_t h[4], l[4];
    pair(x[0], x[1], h[0], l[0]);
    pair(x[2], x[3], h[1], l[1]);
    pair(y[0], y[1], h[2], l[2]);
    pair(y[2], y[3], h[3], l[3]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
  }
};

// K rows of a chunk in the contiguous k order: kf[m][kb] = K[16m + r][32kb +
// 8q .. +7], rows t >= n zero.
__device__ __forceinline__ void load_k_frags(bf16x8 (&kf)[4][4], const uint16_t *kbase, int64_t qk_row, int n,
                                             int lane) {
  const int q4 = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + r16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      kf[m][kb] = (t < n) ? load16_bf16x8(kbase + int64_t(t) * qk_row + 32 * kb + 8 * q4) : zero8();
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two floats -> two float16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Gate scan and UT solve of one chunk by one wave.  In: kf (above), gv / bv
// the g and beta of token `lane` (0 for lanes >= n).  Out: G = G_lane (lanes
// past the end repeat G_{n-1}), Gn = G_{n-1}, and T' as tx[f] (8 float16 per
// lane, f = 0..5).  W is private to the wave for the call.
__device__ __forceinline__ void ut_solve(const bf16x8 (&kf)[4][4], float gv, float bv, int n, UtWork &W,
                                         int lane, u32x4 (&tx)[kTpFrags], float &G, float &Gn) {
  const int q4 = lane >> 4, r16 = lane & 15;
  const SplitK sp;
  auto tile = [&](int mr, int ms) -> float * { return W.L + tri_tile(mr, ms) * kTileF; };

  // ---- gate: inclusive prefix sum over the chunk ---------------------------
  G = gv;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(G, d, 64);
    if (lane >= d) G += o;
  }
  Gn = __shfl(G, n - 1, 64);
  W.Gs[lane] = G * 1.4426950408889634f; // log2(e) G, for exp2 below
  W.Bs[lane] = bv;

  // ---- L = strict_lower(diag(beta) (D * K K^T)), tile by tile --------------
#pragma unroll
  for (int mr = 0; mr < 4; ++mr) {
    const f32x4 gr = *reinterpret_cast<const f32x4 *>(W.Gs + 16 * mr + 4 * q4);
    const f32x4 br = *reinterpret_cast<const f32x4 *>(W.Bs + 16 * mr + 4 * q4);
#pragma unroll
    for (int ms = 0; ms <= mr; ++ms) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(kf[mr][kb], kf[ms][kb], acc);
      const int sc = 16 * ms + r16; // C tile: column s, rows r
      const float gs = W.Gs[sc];
      float *T = tile(mr, ms);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * mr + 4 * q4 + ii;
        T[(4 * q4 + ii) * kTP + r16] = (sc < r) ? br[ii] * __builtin_amdgcn_exp2f(gr[ii] - gs) * acc[ii] : 0.f;
      }
    }
  }

  // ---- diagonal tiles: T_bb = (I + L_bb)^-1, lane 16b + j owns column j of
  // tile (b, b):  T[r][j] = delta_rj - sum_{s<r} L[r][s] T[s][j] ------------
  {
    const int b = lane >> 4, jj = lane & 15;
    float *D = W.L + (b * (b + 1) / 2 + b) * kTileF;
    float t[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float a0 = (rr == jj) ? 1.f : 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      const float *Lr = D + rr * kTP;
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
    // T_bb in place of L_bb (its reads are done)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) D[rr * kTP + jj] = t[rr];
  }

  // ---- off-diagonal tiles of the two diagonal 32x32 blocks (e = 0, 1):
  // T(2e+1, 2e) = -T(2e+1, 2e+1) (L(2e+1, 2e) T(2e, 2e)), 16x16x16 products
  // (A: lane holds row r, columns 4q..4q+3; B: column r, rows 4q..4q+3; C
  // likewise, so P's C fragment is the B operand of the second product) -----
  {
    f32x4 P[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(tile(2 * e + 1, 2 * e) + r16 * kTP + 4 * q4);
      const float *Td = tile(2 * e, 2 * e);
      const f32x4 bcol = {Td[(4 * q4 + 0) * kTP + r16], Td[(4 * q4 + 1) * kTP + r16], Td[(4 * q4 + 2) * kTP + r16],
                          Td[(4 * q4 + 3) * kTP + r16]};
      bf16x4 ah, al, bh, bl;
      sp.four(a, ah, al);
      sp.four(bcol, bh, bl);
      P[e] = mfma16(ah, bh, zero4());
      P[e] = mfma16(ah, bl, P[e]);
      P[e] = mfma16(al, bh, P[e]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(tile(2 * e + 1, 2 * e + 1) + r16 * kTP + 4 * q4);
      bf16x4 ah, al, ph, pl;
      sp.four(a, ah, al);
      sp.four(P[e], ph, pl);
      f32x4 acc = mfma16(ah, ph, zero4());
      acc = mfma16(ah, pl, acc);
      acc = mfma16(al, ph, acc);
      float *To = tile(2 * e + 1, 2 * e);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) To[(4 * q4 + ii) * kTP + r16] = -acc[ii];
    }
  }

  // ---- lower left 32x32 block: T21 = -T22 (L21 T11) -----------------------
  {
    // Pm = L21 T11 (16x16x32 products, contiguous k order: lane holds k =
    // 8q .. 8q+7, inside tile column q / 2).  T11's columns are read from its
    // rows; its upper right tile is zero and not stored.
    const int kt = q4 >> 1, kr0 = 8 * (q4 & 1);
    bf16x8 bh[2], bl[2];
#pragma unroll
    for (int np = 0; np < 2; ++np) {
      const bool nz = (np <= kt); // tile (kt, np) lies on or below the diagonal
      const float *bt = tile(nz ? kt : 1, np) + r16; // (1, 1): any stored tile
      f32x4 x0, x1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = nz ? bt[(kr0 + e) * kTP] : 0.f;
        x1[e] = nz ? bt[(kr0 + 4 + e) * kTP] : 0.f;
      }
      sp.eight(x0, x1, bh[np], bl[np]);
    }
    f32x4 Pm[2][2];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp) {
      const float *ar = tile(2 + mp, kt) + r16 * kTP + kr0;
      bf16x8 ah, al;
      sp.eight(*reinterpret_cast<const f32x4 *>(ar), *reinterpret_cast<const f32x4 *>(ar + 4), ah, al);
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        f32x4 acc = mfma(ah, bh[np], zero4());
        acc = mfma(ah, bl[np], acc);
        Pm[mp][np] = mfma(al, bh[np], acc);
      }
    }
    // T21 = -T22 Pm; Pm's C tiles are the B operand in chain order over the
    // 32 rows of Pm (k = 4q.. in tile 0, 16 + 4q.. in tile 1), and T22's A
    // fragment in chain order is columns 4q.. of its tiles (2 + mt, 2) and
    // (2 + mt, 3) (the latter zero for mt = 0)
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int np = 0; np < 2; ++np)
      sp.eight(Pm[0][np], Pm[1][np], ph[np], pl[np]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(tile(2 + mt, 2) + r16 * kTP + 4 * q4);
      const f32x4 a1 = (mt == 1) ? *reinterpret_cast<const f32x4 *>(tile(3, 3) + r16 * kTP + 4 * q4) : zero4();
      bf16x8 ah, al;
      sp.eight(a0, a1, ah, al);
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        f32x4 acc = mfma(ah, ph[np], zero4());
        acc = mfma(ah, pl[np], acc);
        acc = mfma(al, ph[np], acc);
        float *To = tile(2 + mt, np);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) To[(4 * q4 + ii) * kTP + r16] = -acc[ii];
      }
    }
  }

  // ---- T' = T diag(beta), float16, in fragment order ----------------------
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (2 * kb > mt) continue;
      const int s0 = 32 * kb + 4 * q4;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(tile(mt, 2 * kb) + r16 * kTP + 4 * q4) *
                      *reinterpret_cast<const f32x4 *>(W.Bs + s0);
      u32x4 out = {cvt_pk_f16(a[0], a[1]), cvt_pk_f16(a[2], a[3]), 0u, 0u};
      if (2 * kb + 1 <= mt) { // else the second four columns lie above the diagonal
        const f32x4 b = *reinterpret_cast<const f32x4 *>(tile(mt, 2 * kb + 1) + r16 * kTP + 4 * q4) *
                        *reinterpret_cast<const f32x4 *>(W.Bs + s0 + 16);
        out[2] = cvt_pk_f16(b[0], b[1]);
        out[3] = cvt_pk_f16(b[2], b[3]);
      }
      tx[tri_frag(mt, kb)] = out;
    }
}

} // namespace gdn
