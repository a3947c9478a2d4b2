// gdn_ut_solve.h -- the per-chunk gate scan and UT solve, one wave per
// (chunk, v-head), of chunk_cumsum_recompute_wu.  Its exact bf16 hi/lo split
// (SplitK) has the same form as the spine's (split_tiles).
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 1: the chunk-local cumulative log-gate gc and the WY/UT solves
// (I+L) U = beta V, (I+L) W = beta exp(gc) K, with L sharing the key Gram
// matrix's buffer (comment above smem_wu).  For the chunk's n <= 64 tokens
// (lanes past the sequence end carry g = beta = 0):
//   G_r    = sum_{j<=r} g_j
//   L[r,s] = beta_r exp(G_r - G_s) (k_r . k_s)        (s < r, else 0)
//   T'     = (I + L)^-1 diag(beta)                     (the UT transform)
// so that U = T' V and W = T' diag(exp(G)) K.  With the keys normalised to
// unit length (k_r / |k_r|), K stays the exact bf16 operand of the Gram and
// the row scales sk_r = 1/|k_r| multiply its result in float32:
//   L[r,s] = beta_r exp(G_r - G_s) sk_r sk_s (k_r . k_s).
// T = (I+L)^-1 by blocks: for a unit lower-triangular [[A, 0], [C, D]], the
// inverse is [[A^-1, 0], [-D^-1 C A^-1, D^-1]].
//   * lane t scans g;
//   * the lower 10 16x16 tiles of K K^T on bf16 MFMA (K is exact in bf16) ->
//     L in registers, its four diagonal tiles also in LDS;
//   * the four diagonal 16x16 tiles of T by f32 forward substitution, one lane
//     per column of each (<= 120 FMAs per lane);
//   * the off-diagonal tiles of the two diagonal 32x32 blocks, then the lower
//     left 32x32 block, by the formula above on MFMA, transposed, every
//     operand split into bf16 hi + lo (three products each, ~2^-17 relative
//     error);
//   * T' = T diag(beta), split into bf16 hi + lo (hi = bf16(x), lo =
//     bf16(x - hi): ~2^-17 relative, what the spine's products of T' with the
//     split R use), in the A-operand fragment
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

// LDS tiles: the four diagonal 16x16 tiles of L, overwritten by those of T,
// and T's tile (1, 0); row-major with a pitch of kTP floats, kTileF floats
// apart.  The pitch puts the 4 rows x 16 columns a wave writes from a C
// fragment, or reads as a column fragment, in 64 distinct banks; the extra 4
// floats per tile put the four diagonal tiles, which the substitution reads at
// once, in different banks.  The off-diagonal tiles of L never leave the
// registers they are formed in.
constexpr int kTP = 20;
constexpr int kTileF = 16 * kTP + 4;
__host__ __device__ constexpr int tri_tile(int mr, int ms) { return mr * (mr + 1) / 2 + ms; }

// LDS workspace of one solving wave (7.2 KB).
struct __align__(16) UtWork {
  float D[5 * kTileF]; // tiles 0..3: (b, b); tile 4: T(1, 0)
  float Gs[kChunk];    // log2(e) G_t, for exp2
  float Bs[kChunk];    // beta_t
  float Sk[kChunk];    // 1/|k_t| (normalised keys only)
};

// Sum of squares of the eight bf16 values of x, added to acc (four bf16 dot
// products with float32 accumulation).  Each 32-bit word is copied to a
// scalar before the bit cast: hipcc compiles a bit cast of a vector element
// w[e] to element 0 for every e.
__device__ __forceinline__ float sumsq8(const bf16x8 &x, float acc) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t we = w[e];
    const bf16x2 p = __builtin_bit_cast(bf16x2, we);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// 1/|x| of the chunk row `lane` from row fragments f[m][kb] (as load_k_frags
// leaves them: lane 16q + r holds row 16m + r, columns 32kb + 8q .. +7): the
// row's 128 squares are summed over a lane's 32 values, then over the four
// lanes q = 0..3 that share r.  A row whose squares sum to 0 (or underflow)
// gets 0, so that the normalised row is 0.
__device__ __forceinline__ float inv_row_norm(const bf16x8 (&f)[4][4], int lane) {
  float ps[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float a = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) a = sumsq8(f[m][kb], a);
    a += __shfl_xor(a, 16, 64);
    a += __shfl_xor(a, 32, 64);
    ps[m] = a;
  }
  const int q4 = lane >> 4;
  const float own = q4 == 0 ? ps[0] : q4 == 1 ? ps[1] : q4 == 2 ? ps[2] : ps[3];
  return own > 0.f ? rsqrtf(own) : 0.f;
}

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
// 8q .. +7].  Rows t >= n repeat row n-1: they only meet beta = 0 (their rows
// of L) or the strict lower mask (their columns), so T' does not depend on
// them, and the loads carry no condition that would make them wait on one
// another.
__device__ __forceinline__ void load_k_frags(bf16x8 (&kf)[4][4], const uint16_t *kbase, int64_t qk_row, int n,
                                             int lane) {
  const int q4 = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = min(16 * m + r16, n - 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kf[m][kb] = load16_bf16x8(kbase + int64_t(t) * qk_row + 32 * kb + 8 * q4);
  }
}

// Gate scan and UT solve of one chunk by one wave.  In: kf (above), gv / bv
// the g and beta of token `lane` (0 for lanes >= n), skv its key scale
// 1/|k_lane| (read only with kNorm).  Out: G = G_lane (lanes past the end
// repeat G_{n-1}), Gn = G_{n-1}, and T' as tx[f] (bf16 hi, 8 per lane,
// f = 0..5) and tx[6 + f] (bf16 lo).  W is private to the wave for the call.
template <bool kNorm>
__device__ __forceinline__ void ut_solve(const bf16x8 (&kf)[4][4], float gv, float bv, float skv, int n,
                                         UtWork &W, int lane, u32x4 (&tx)[2 * kTpFrags], float &G, float &Gn) {
  const int q4 = lane >> 4, r16 = lane & 15;
  const SplitK sp;
  auto dt = [&](int b) -> float * { return W.D + b * kTileF; };
  // rows 4q .. 4q+3 of column r of an LDS tile (a C, or B, fragment)
  auto col4 = [&](const float *T) -> f32x4 {
    return f32x4{T[(4 * q4) * kTP + r16], T[(4 * q4 + 1) * kTP + r16], T[(4 * q4 + 2) * kTP + r16],
                 T[(4 * q4 + 3) * kTP + r16]};
  };
  // columns 4q .. 4q+3 of row r of an LDS tile (an A fragment)
  auto row4 = [&](const float *T) -> f32x4 { return *reinterpret_cast<const f32x4 *>(T + r16 * kTP + 4 * q4); };

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
  if (kNorm) W.Sk[lane] = skv;

  // ---- L = strict_lower(diag(beta) (D * K K^T)) as C fragments (lane: column
  // 16ms + r, rows 16mr + 4q .. +3); the diagonal tiles go to LDS -----------
  f32x4 lc[10];
#pragma unroll
  for (int mr = 0; mr < 4; ++mr) {
    const f32x4 gr = *reinterpret_cast<const f32x4 *>(W.Gs + 16 * mr + 4 * q4);
    f32x4 br = *reinterpret_cast<const f32x4 *>(W.Bs + 16 * mr + 4 * q4);
    if (kNorm) br *= *reinterpret_cast<const f32x4 *>(W.Sk + 16 * mr + 4 * q4); // beta_r sk_r
#pragma unroll
    for (int ms = 0; ms <= mr; ++ms) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma(kf[mr][kb], kf[ms][kb], acc);
      const int sc = 16 * ms + r16;
      const float gs = W.Gs[sc];
      if (kNorm) acc *= W.Sk[sc]; // sk_s
      f32x4 l;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * mr + 4 * q4 + ii;
        l[ii] = (sc < r) ? br[ii] * __builtin_amdgcn_exp2f(gr[ii] - gs) * acc[ii] : 0.f;
      }
      if (ms == mr) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) dt(mr)[(4 * q4 + ii) * kTP + r16] = l[ii];
      } else {
        lc[tri_tile(mr, ms)] = l;
      }
    }
  }

  // ---- diagonal tiles: T_bb = (I + L_bb)^-1, lane 16b + j owns column j of
  // tile (b, b):  T[r][j] = delta_rj - sum_{s<r} L[r][s] T[s][j] ------------
  {
    const int b = lane >> 4, jj = lane & 15;
    float *D = dt(b);
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

  // The remaining blocks are formed transposed: a C fragment read as an A
  // operand is the transpose of its tile, so L's off-diagonal tiles serve as
  // A operands where they are, and each result comes out with a lane holding
  // four consecutive columns of one row -- the order of T''s fragments.

  // ---- off-diagonal tiles of the two diagonal 32x32 blocks (e = 0, 1):
  // T(2e+1, 2e)^T = -T(2e, 2e)^T (L(2e+1, 2e)^T T(2e+1, 2e+1)^T) -------------
  f32x4 Rt[2]; // Rt[e]: lane holds T(2e+1, 2e)[r][4q .. 4q+3]
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    bf16x4 ah, al, bh, bl;
    sp.four(lc[tri_tile(2 * e + 1, 2 * e)], ah, al);  // L(2e+1, 2e)^T
    sp.four(row4(dt(2 * e + 1)), bh, bl);             // T(2e+1, 2e+1)^T
    f32x4 Q = mfma16(ah, bh, zero4());
    Q = mfma16(ah, bl, Q);
    Q = mfma16(al, bh, Q);
    sp.four(col4(dt(2 * e)), ah, al);                 // T(2e, 2e)^T
    bf16x4 qh, ql;
    sp.four(Q, qh, ql);
    f32x4 acc = mfma16(ah, qh, zero4());
    acc = mfma16(ah, ql, acc);
    acc = mfma16(al, qh, acc);
    Rt[e] = -acc;
  }
  // T(1, 0) to LDS: its columns are an operand below
  *reinterpret_cast<f32x4 *>(dt(4) + r16 * kTP + 4 * q4) = Rt[0];

  // ---- lower left 32x32 block: T21^T = -T11^T (L21^T T22^T), 16x16x32
  // products in chain order (k = 4q.. in the first tile, 16 + 4q.. in the
  // second) ------------------------------------------------------------------
  // Q2[mp][np] = L21^T T22^T; A: L21^T row tile mp = L's tiles (2, mp), (3, mp)
  // as C fragments; B: T22 rows 16np + r, columns 4q.. of its two column tiles
  bf16x8 t22h[2], t22l[2];
  sp.eight(row4(dt(2)), zero4(), t22h[0], t22l[0]);
  sp.eight(Rt[1], row4(dt(3)), t22h[1], t22l[1]);
  f32x4 Q2[2][2];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    bf16x8 ah, al;
    sp.eight(lc[tri_tile(2, mp)], lc[tri_tile(3, mp)], ah, al);
#pragma unroll
    for (int np = 0; np < 2; ++np) {
      f32x4 acc = mfma(ah, t22h[np], zero4());
      acc = mfma(ah, t22l[np], acc);
      Q2[mp][np] = mfma(al, t22h[np], acc);
    }
  }
  // T21^T[mt][np] = -T11^T Q2: A: T11 columns 16mt + r, rows 4q.. of its two
  // row tiles (T(0, mt) and T(1, mt); T(0, 1) = 0); B: Q2's C tiles
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int np = 0; np < 2; ++np) sp.eight(Q2[0][np], Q2[1][np], qh[np], ql[np]);
  f32x4 T21t[2][2]; // lane holds T21[16np + r][16mt + 4q .. +3]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    bf16x8 ah, al;
    sp.eight(mt == 0 ? col4(dt(0)) : zero4(), col4(mt == 0 ? dt(4) : dt(1)), ah, al);
#pragma unroll
    for (int np = 0; np < 2; ++np) {
      f32x4 acc = mfma(ah, qh[np], zero4());
      acc = mfma(ah, ql[np], acc);
      acc = mfma(al, qh[np], acc);
      T21t[mt][np] = -acc;
    }
  }

  // ---- T' = T diag(beta), bf16 hi + lo, in fragment order: fragment (mt, kb)
  // is row 16mt + r, columns 32kb + 4q .. and 32kb + 16 + 4q .. -------------
  auto emit = [&](int f, int kb, const f32x4 &a, const f32x4 &b, bool two) {
    const int s0 = 32 * kb + 4 * q4;
    const f32x4 x = a * *reinterpret_cast<const f32x4 *>(W.Bs + s0);
    uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
    sp.pair(x[0], x[1], hi[0], lo[0]);
    sp.pair(x[2], x[3], hi[1], lo[1]);
    if (two) {
      const f32x4 y = b * *reinterpret_cast<const f32x4 *>(W.Bs + s0 + 16);
      sp.pair(y[0], y[1], hi[2], lo[2]);
      sp.pair(y[2], y[3], hi[3], lo[3]);
    }
    tx[f] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    tx[kTpFrags + f] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  };
  emit(tri_frag(0, 0), 0, row4(dt(0)), zero4(), false);
  emit(tri_frag(1, 0), 0, Rt[0], row4(dt(1)), true);
  emit(tri_frag(2, 0), 0, T21t[0][0], T21t[1][0], true);
  emit(tri_frag(3, 0), 0, T21t[0][1], T21t[1][1], true);
  emit(tri_frag(2, 1), 1, row4(dt(2)), zero4(), false);
  emit(tri_frag(3, 1), 1, Rt[1], row4(dt(3)), true);
}

} // namespace gdn
