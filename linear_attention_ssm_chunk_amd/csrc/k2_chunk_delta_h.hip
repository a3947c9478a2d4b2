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
//
// The dv columns of h evolve independently, so the state is split into
// 16-column strips (the page's DV-block split, tc_vblock comment).  A
// workgroup covers S strips of one chain (S = 1, 2 or 4, chosen so the grid
// fills the chip: few long chains get more workgroups each):
//   * waves 0..S-1 (compute): one strip each for the whole pass.  The strip
//     lives in MFMA accumulators; in the chain k order those registers are the
//     B operand of K h directly, and so are the C tiles of R = V - e^G K h (for
//     T' R) and of uc (for K^T uc): the dependent chain never leaves registers;
//   * waves S..S+3 (loaders), two pairs: the pair that owns chunk c+1 copies
//     the K, K^T and T' fragments, the decays and the workgroup's columns of
//     V (transposed, so a lane reads its four rows of a tile at once), fetched
//     two steps earlier, into the free half of a double-buffered LDS stage,
//     then fetches chunk c+3.  Fragment accesses on both sides are
//     lane-contiguous (fragment order from stage 1).
// One barrier per chunk.
// Precision: h is float32 between chunks; h, R and the decayed uc are split
// into bf16 hi+lo for the products that feed the state (K is exact in bf16, T'
// arrives split), so every product keeps ~2^-17 relative error with bf16 MFMA
// and float32 accumulation.
//
// Workgroup order: all workgroups that read one k-head's chunk tiles (its r
// v-heads x column groups) get the same blockIdx.x % 8, so that on a
// round-robin XCD dispatch they share one XCD's L2.
#include "gdn_device.h"

namespace gdn {

constexpr int kVPitch = 68; // 136-byte columns: lanes 16 columns apart hit different banks
struct Stage {
  u32x4 kn[16 * 64];    // K, A operand of K h: fragment (mt, kb), chain order over dk
  u32x4 kt[16 * 64];    // K^T, A operand of K^T uc: fragment (m, kb), chain order over t
  u32x4 tp[2 * 8 * 64]; // T' fragments: 8 hi, then 8 lo
  float dec[2 * kChunk]; // exp(G_t), exp(G_{n-1} - G_t)
  uint16_t vn[kChunk * kVPitch]; // V transposed, [column][t], the workgroup's <= 64 columns
};

// Split two C tiles (a k block of 32 rows, chain order) into hi / lo bf16
// fragments, overwriting the tiles.  hi = bf16(x); x - hi is exact in float32
// and comes from one bf16 dot product per element, (hi0, hi1) . (-1, 0) + x0,
// with the constant pairs in registers m0, m1 (an inline constant would be read
// as the float32 -1.0).  The four pairs go side by side so that no instruction
// waits on the one before it.
__device__ __forceinline__ void split_tiles(f32x4 &t0, f32x4 &t1, uint32_t m0, uint32_t m1, bf16x8 &hi, bf16x8 &lo) {
  uint32_t h[4], l[4];
  float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = cvt_pk(x[2 * e], x[2 * e + 1]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 h2 = __builtin_bit_cast(bf16x2, h[e]);
    x[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(h2, __builtin_bit_cast(bf16x2, m0), x[2 * e], false);
    x[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(h2, __builtin_bit_cast(bf16x2, m1), x[2 * e + 1], false);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) l[e] = cvt_pk(x[2 * e], x[2 * e + 1]);
  hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

template <int kStrips>
__global__ __launch_bounds__((kStrips + 4) * 64) void chunk_delta_h(Params p) {
  constexpr int kGroups = 8 / kStrips; // workgroups per chain
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

  __shared__ Stage st[2];

  // =========================== loader waves ===============================
  if (wave >= kStrips) {
    const int pair = (wave - kStrips) >> 1;            // owns chunks c with c % 2 == pair
    const int lt = ((wave - kStrips) & 1) * 64 + lane; // 0..127 within the pair
    u32x4 pk[8], pt[8], pp[8], pv[kStrips];
    float pd = 0.f;
    // V: 16-byte pieces of the workgroup's 16 * kStrips columns, kStrips per lane
    constexpr int kPieces = 2 * kStrips; // per row
    const uint16_t *vcols = p.v + int64_t(h) * kDim + cg * 16 * kStrips;
    auto fetch = [&](int c) {
      const u32x4 *ksrc = reinterpret_cast<const u32x4 *>(
          p.kfr + (s.chunk0 * p.nk + int64_t(kh) * s.nchunks + c) * (2 * 16 * 64 * 8));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pk[jj] = ksrc[lt + 128 * jj];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pt[jj] = ksrc[1024 + lt + 128 * jj];
      const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(p.tp + slot_of(p, s, h, c) * (2 * 8 * 64 * 8));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pp[jj] = tsrc[lt + 128 * jj];
      pd = p.dec[slot_of(p, s, h, c) * 2 * kChunk + lt];
      const int nn = min(kChunk, s.len - c * kChunk);
      const uint16_t *vsrc = vcols + (s.tok0 + int64_t(c) * kChunk) * p.v_row;
#pragma unroll
      for (int jj = 0; jj < kStrips; ++jj) {
        const int piece = lt + 128 * jj, row = piece / kPieces;
        // rows past the sequence end repeat its last row (they meet zero
        // columns of T' only)
        pv[jj] = *reinterpret_cast<const u32x4 *>(vsrc + int64_t(min(row, nn - 1)) * p.v_row + 8 * (piece % kPieces));
      }
    };
    auto stash = [&](Stage &S) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) S.kn[lt + 128 * jj] = pk[jj];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) S.kt[lt + 128 * jj] = pt[jj];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) S.tp[lt + 128 * jj] = pp[jj];
      S.dec[lt] = pd;
#pragma unroll
      for (int jj = 0; jj < kStrips; ++jj) {
        const int piece = lt + 128 * jj, row = piece / kPieces;
        uint16_t *dst = S.vn + (8 * (piece % kPieces)) * kVPitch + row; // column 8 * (piece % kPieces)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dst[e * kVPitch] = uint16_t(e & 1 ? pv[jj][e >> 1] >> 16 : pv[jj][e >> 1] & 0xFFFFu);
      }
    };

    // prologue: chunk `pair` is fetched now; pair 0 also stages chunk 0 and
    // fetches chunk 2 before the first barrier
    if (pair < s.nchunks) fetch(pair);
    if (pair == 0) {
      stash(st[0]);
      if (2 < s.nchunks) fetch(2);
    }
    __syncthreads();
    for (int c = 0; c < s.nchunks; ++c) {
      // the pair owning chunk c+1 stages it into the half compute is not reading
      if (((c + 1) & 1) == pair && c + 1 < s.nchunks) {
        stash(st[(c + 1) & 1]);
        if (c + 3 < s.nchunks) fetch(c + 3);
      }
      __syncthreads();
    }
    return;
  }

  // =========================== compute waves ==============================
  const int colw = cg * 16 * kStrips + 16 * wave; // this wave's strip
  float *hp = state_of(p, i, h);
  f32x4 H[8]; // H[m][ii] = h[16m + 4q + ii][colw + r16]
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) H[m][ii] = hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16];

  // bf16 pairs (-1, 0) and (0, -1) for split_tiles, kept in registers
  uint32_t m0 = 0x0000BF80u, m1 = 0xBF800000u;
  asm volatile("" : "+v"(m0));
  asm volatile("" : "+v"(m1));
  const int vcol = 16 * wave + r16; // column within the workgroup's staged V

  __syncthreads(); // chunk 0 staged

  for (int c = 0; c < s.nchunks; ++c) {
    const Stage &S = st[c & 1];
    const int64_t sl = slot_of(p, s, h, c);
    // V of this chunk at the lane's C positions: rows 16mt + 4q .. +3, one
    // 8-byte read per tile
    uint32_t vv[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const u32x2 v = *reinterpret_cast<const u32x2 *>(S.vn + vcol * kVPitch + 16 * mt + 4 * q4);
      vv[mt][0] = v[0];
      vv[mt][1] = v[1];
    }

    // h -> hi/lo bf16, chain order over dk; bf16(h) is also the entry state
    bf16x8 Hh[4], Hl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) chain_split(H[2 * kb], H[2 * kb + 1], Hh[kb], Hl[kb]);
    {
      // S_c = h^T: row dv = colw + r16, dk = 32kb + 4q .. +3 and +16
      uint16_t *sdst = p.s_entry + sl * (kDim * kDim) + (colw + r16) * kDim + 4 * q4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 hv = __builtin_bit_cast(u32x4, Hh[kb]);
        *reinterpret_cast<u32x2 *>(sdst + 32 * kb) = u32x2{hv[0], hv[1]};
        *reinterpret_cast<u32x2 *>(sdst + 32 * kb + 16) = u32x2{hv[2], hv[3]};
      }
    }

    // R = V - diag(exp(G)) K h   (C tile mt: column colw + r16, rows t = 16mt + 4q .. +3)
    // Consecutive products go to different accumulators (k block outer).
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 ka[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ka[mt] = __builtin_bit_cast(bf16x8, S.kn[(mt * 4 + kb) * 64 + lane]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(ka[mt], Hh[kb], acc[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(ka[mt], Hl[kb], acc[mt]);
    }
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 eg = *reinterpret_cast<const f32x4 *>(S.dec + 16 * mt + 4 * q4);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t pr = vv[mt][ii >> 1];
        const float v = __builtin_bit_cast(float, (ii & 1) ? (pr & 0xFFFF0000u) : (pr << 16));
        R[mt][ii] = v - eg[ii] * acc[mt][ii];
      }
    }
    bf16x8 Rh[2], Rl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_tiles(R[2 * kb], R[2 * kb + 1], m0, m1, Rh[kb], Rl[kb]);

    // uc = T' R  (T' is lower triangular: fragment (mt, 1) is zero for mt < 2)
    f32x4 D[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 th[4], tl[4];
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) {
        th[mt] = __builtin_bit_cast(bf16x8, S.tp[(mt * 2 + kb) * 64 + lane]);
        tl[mt] = __builtin_bit_cast(bf16x8, S.tp[8 * 64 + (mt * 2 + kb) * 64 + lane]);
      }
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(th[mt], Rh[kb], D[mt]);
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(th[mt], Rl[kb], D[mt]);
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(tl[mt], Rh[kb], D[mt]);
    }

    // uc store, transposed: uc[slot][dv][t .. t+3]
    {
      uint16_t *udst = p.uc + sl * (kDim * kChunk) + (colw + r16) * kChunk + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<u32x2 *>(udst + 16 * mt) = pack4_bf16(D[mt][0], D[mt][1], D[mt][2], D[mt][3]);
    }

    // h <- exp(G_n) h + K^T diag(exp(G_n - G)) uc
    const float en = S.dec[kChunk - 1]; // exp(G) of the last row = exp(G_n): rows past the end repeat it
#pragma unroll
    for (int m = 0; m < 8; ++m) H[m] *= en;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) D[mt] *= *reinterpret_cast<const f32x4 *>(S.dec + kChunk + 16 * mt + 4 * q4);
    bf16x8 Dh[2], Dl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_tiles(D[2 * kb], D[2 * kb + 1], m0, m1, Dh[kb], Dl[kb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 ka[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) ka[m] = __builtin_bit_cast(bf16x8, S.kt[(m * 2 + kb) * 64 + lane]);
#pragma unroll
      for (int m = 0; m < 8; ++m) H[m] = mfma(ka[m], Dh[kb], H[m]);
#pragma unroll
      for (int m = 0; m < 8; ++m) H[m] = mfma(ka[m], Dl[kb], H[m]);
    }

    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16] = H[m][ii];
}

namespace {
int compute_units() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <int kStrips>
hipError_t launch_with(const Params &p, hipStream_t stream) {
  const int r = p.nv / p.nk;
  const int kgroups = p.B * p.nk;
  const int blocks = 8 * ((kgroups + 7) / 8) * r * (8 / kStrips);
  hipLaunchKernelGGL(chunk_delta_h<kStrips>, dim3(blocks), dim3((kStrips + 4) * 64), 0, stream, p);
  return hipGetLastError();
}
} // namespace

// Strips per workgroup: the fewest that keep the grid within one workgroup per
// compute unit (the stage's LDS allows one per CU), so chains with few heads
// spread over more CUs and many chains share LDS-staged tiles.
hipError_t launch_stage2(const Params &p, hipStream_t stream) {
  const long chains = long(p.B) * p.nv;
  const int cus = compute_units();
  if (chains * 8 <= cus) return launch_with<1>(p, stream);
  if (chains * 4 <= cus) return launch_with<2>(p, stream);
  return launch_with<4>(p, stream);
}

} // namespace gdn
