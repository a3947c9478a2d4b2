// Stage 2: chunk_delta_h, the serial float32 state spine.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 2: one pass over the chunks of each (sequence, v-head) that emits the
// per-chunk entry states and the corrected values uc, and updates h_state in
// place.  Per chunk, with h the entry state (stored [dk][dv], float32) and T'
// the UT transform from stage 1:
//   S_entry[c] = bf16(h^T)                                  ([dv][dk])
//   uc         = U - W h = T' (V - diag(exp(G)) K h)        (stored bf16, [dv][t])
//   h         <- exp(G_n) h + K^T diag(exp(G_n - G)) uc     (G_n: last token)
// The dv columns of h evolve independently, so the state is split into
// 16-column strips (the page's DV-block split, tc_vblock comment): one wave
// owns one strip for the whole pass; a workgroup holds 4 strips, two
// workgroups per chain.  The strip lives in MFMA accumulators; in the chain k
// order those registers are the B operand of K h directly, and so are the C
// tiles of K h (for T' R) and of uc (for K^T uc) -- the chain never leaves
// registers.  K, V, T' and the decays of chunk c+1 are fetched into registers
// while chunk c computes and written to the other half of a double-buffered
// LDS stage: one barrier per chunk.
// Precision: h is float32 between chunks; h, R = V - e^G K h and the decayed
// uc are split into bf16 hi+lo for the products that feed the state (K is
// exact in bf16, T' arrives split), so every product keeps ~2^-17 relative
// error with bf16 MFMA and float32 accumulation.
//
// Workgroup order: all workgroups that read one k-head's chunk tiles (its r
// v-heads x 2 column groups) get the same blockIdx.x % 8, so that on a
// round-robin XCD dispatch they share one XCD's L2.
#include "gdn_device.h"

namespace gdn {

constexpr int kStrips = 4;           // waves (16-column strips) per workgroup
constexpr int kCols = 16 * kStrips;  // state columns per workgroup
constexpr int kGroups = kDim / kCols; // workgroups per chain
constexpr int kKP = 132;             // natural K tile pitch (bf16): 264 B rows
constexpr int kVP = 68;              // V tile pitch (bf16): 136 B rows

struct Stage {
  uint16_t kn[kChunk * kKP];          // K[t][dk]
  unsigned char kt[kDim * kChunk * 2]; // K^T, swizzled (kt_off)
  uint16_t vs[kChunk * kVP];          // V[t][col0 .. col0+63]
  u32x4 tp[8 * 64 * 2];               // T' fragments (hi, lo)
  float dec[2 * kChunk];              // exp(G_t), exp(G_{n-1} - G_t)
};

// Byte offset of K^T[d][t] (t a multiple of 4): rows of 64 tokens (128 B) in
// 16-byte granules, granule index XOR-swizzled with f(d) = (d ^ d>>3) & 7 so
// that the transposing stores (16 rows 8 apart) and the fragment loads (16
// consecutive rows) both spread over all banks.
__device__ __forceinline__ int kt_off(int d, int t) {
  const int f = (d ^ (d >> 3)) & 7;
  return d * 128 + ((((t >> 3) ^ f) & 7) << 4) + ((t >> 2) & 1) * 8;
}

__global__ __launch_bounds__(kThreads) void chunk_delta_h(Params p) {
  // ---- which (sequence, v-head, column group) ----------------------------
  const int r = p.nv / p.nk;
  const int b = blockIdx.x;
  const int idx = b >> 3;
  const int kgroup = (b & 7) + 8 * (idx / (r * kGroups)); // (sequence, k-head)
  if (kgroup >= p.B * p.nk) return;
  const int j = (idx / kGroups) % r, cg = idx % kGroups;
  const int i = kgroup / p.nk, kh = kgroup % p.nk;
  const int h = kh * r + j;
  const Seq s = seq_of(p, i);
  if (!s.ok || s.nchunks == 0) return; // length 0: the state is left as it is

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int col0 = cg * kCols;       // workgroup's first column
  const int colw = col0 + 16 * wave; // this wave's strip
  float *hp = state_of(p, i, h);

  __shared__ Stage st[2];

  // state strip: H[m][ii] = h[16m + 4q + ii][colw + r16]
  f32x4 H[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) H[m][ii] = hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16];

  // ---- prefetch registers --------------------------------------------------
  const int dg = tid & 15, tg = tid >> 4; // K: 8 columns x 4 tokens per thread
  u32x4 kreg[4], vreg[2], treg[4];
  float dreg = 0.f;
  auto fetch = [&](int c) {
    const int64_t sl = slot_of(p, s, h, c);
    const int n = min(kChunk, s.len - c * kChunk);
    const int64_t row0 = s.tok0 + int64_t(c) * kChunk;
    const uint16_t *ksrc = p.k + row0 * p.qk_row + int64_t(kh) * kDim + 8 * dg;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int t = 4 * tg + jj;
      kreg[jj] = (t < n) ? *reinterpret_cast<const u32x4 *>(ksrc + int64_t(t) * p.qk_row) : u32x4{0u, 0u, 0u, 0u};
    }
    const uint16_t *vsrc = p.v + row0 * p.v_row + int64_t(h) * kDim + col0 + 8 * (tid & 7);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int t = (tid >> 3) + 32 * jj;
      vreg[jj] = (t < n) ? *reinterpret_cast<const u32x4 *>(vsrc + int64_t(t) * p.v_row) : u32x4{0u, 0u, 0u, 0u};
    }
    const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(p.tp + sl * (8 * 64 * 16));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) treg[jj] = tsrc[tid + kThreads * jj];
    if (tid < 2 * kChunk) dreg = p.dec[sl * 2 * kChunk + tid];
  };
  auto stash = [&](Stage &S) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 *dst = reinterpret_cast<u32x2 *>(S.kn + (4 * tg + jj) * kKP + 8 * dg);
      dst[0] = u32x2{kreg[jj][0], kreg[jj][1]};
      dst[1] = u32x2{kreg[jj][2], kreg[jj][3]};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t x0 = (kreg[0][e >> 1] >> sh) & 0xFFFFu, x1 = (kreg[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t x2 = (kreg[2][e >> 1] >> sh) & 0xFFFFu, x3 = (kreg[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<u32x2 *>(S.kt + kt_off(8 * dg + e, 4 * tg)) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      u32x2 *dst = reinterpret_cast<u32x2 *>(S.vs + ((tid >> 3) + 32 * jj) * kVP + 8 * (tid & 7));
      dst[0] = u32x2{vreg[jj][0], vreg[jj][1]};
      dst[1] = u32x2{vreg[jj][2], vreg[jj][3]};
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) S.tp[tid + kThreads * jj] = treg[jj];
    if (tid < 2 * kChunk) S.dec[tid] = dreg;
  };

  fetch(0);
  stash(st[0]);
  __syncthreads();

  for (int c = 0; c < s.nchunks; ++c) {
    Stage &S = st[c & 1];
    const int n = min(kChunk, s.len - c * kChunk);
    const int64_t sl = slot_of(p, s, h, c);
    if (c + 1 < s.nchunks) fetch(c + 1);

    // entry state S_c = h^T: the strip's lane holds 4 consecutive dk of one dv
    {
      uint16_t *sdst = p.s_entry + sl * (kDim * kDim) + (colw + r16) * kDim + 4 * q4;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        *reinterpret_cast<u32x2 *>(sdst + 16 * m) = pack4_bf16(H[m][0], H[m][1], H[m][2], H[m][3]);
    }

    // h -> hi/lo bf16, chain order over dk
    bf16x8 Hh[4], Hl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) chain_split(H[2 * kb], H[2 * kb + 1], Hh[kb], Hl[kb]);

    // R = V - diag(exp(G)) K h   (C tile mt: column colw + r16, rows t = 16mt + 4q .. +3)
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t *kr = S.kn + (16 * mt + r16) * kKP + 4 * q4;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 ka = join8(*reinterpret_cast<const u32x2 *>(kr + 32 * kb),
                                *reinterpret_cast<const u32x2 *>(kr + 32 * kb + 16));
        acc = mfma(ka, Hh[kb], acc);
        acc = mfma(ka, Hl[kb], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = 16 * mt + 4 * q4 + ii;
        const float vv = bf16_bits_to_f32(S.vs[t * kVP + 16 * wave + r16]);
        R[mt][ii] = vv - S.dec[t] * acc[ii];
      }
    }
    bf16x8 Rh[2], Rl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) chain_split(R[2 * kb], R[2 * kb + 1], Rh[kb], Rl[kb]);

    // uc = T' R  (T' is lower triangular: fragment (mt, 1) is zero for mt < 2)
    f32x4 D[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && mt < 2) continue;
        const u32x4 *tf = S.tp + ((mt * 2 + kb) * 64 + lane) * 2;
        const bf16x8 th = __builtin_bit_cast(bf16x8, tf[0]);
        const bf16x8 tl = __builtin_bit_cast(bf16x8, tf[1]);
        acc = mfma(th, Rh[kb], acc);
        acc = mfma(th, Rl[kb], acc);
        acc = mfma(tl, Rh[kb], acc);
      }
      D[mt] = acc;
    }

    // uc store, transposed: uc[slot][dv][t .. t+3]
    {
      uint16_t *udst = p.uc + sl * (kDim * kChunk) + (colw + r16) * kChunk + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<u32x2 *>(udst + 16 * mt) = pack4_bf16(D[mt][0], D[mt][1], D[mt][2], D[mt][3]);
    }

    // h <- exp(G_n) h + K^T diag(exp(G_n - G)) uc
    const float en = S.dec[n - 1];
#pragma unroll
    for (int m = 0; m < 8; ++m) H[m] *= en;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) D[mt][ii] *= S.dec[kChunk + 16 * mt + 4 * q4 + ii];
    bf16x8 Dh[2], Dl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) chain_split(D[2 * kb], D[2 * kb + 1], Dh[kb], Dl[kb]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int d = 16 * m + r16;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(S.kt + kt_off(d, 32 * kb + 4 * q4));
        const u32x2 y = *reinterpret_cast<const u32x2 *>(S.kt + kt_off(d, 32 * kb + 16 + 4 * q4));
        const bf16x8 ka = join8(x, y);
        H[m] = mfma(ka, Dh[kb], H[m]);
        H[m] = mfma(ka, Dl[kb], H[m]);
      }
    }

    if (c + 1 < s.nchunks) stash(st[(c + 1) & 1]);
    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16] = H[m][ii];
}

hipError_t launch_stage2(const Params &p, hipStream_t stream) {
  const int r = p.nv / p.nk;
  const int kgroups = p.B * p.nk;
  const int blocks = 8 * ((kgroups + 7) / 8) * r * kGroups;
  hipLaunchKernelGGL(chunk_delta_h, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
