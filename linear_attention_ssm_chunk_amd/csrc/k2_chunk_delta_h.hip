// Stage 2: chunk_delta_h, the serial float32 state spine.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stage 2: one pass over the chunks of each (sequence, v-head) that emits the
// per-chunk entry states and the corrected values uc, and updates h_state in
// place.  Per chunk, with h the entry state ([dk][dv], float32):
//   S_entry[c] = bf16(h)
//   uc         = U - W h                        (stored bf16, [dv][token])
//   h         <- exp(G_n) h + K^T diag(exp(G_n - G)) uc      (G_n: last token)
// The dv columns of h evolve independently, so the state is split into
// 16-column strips (the page's DV-block split, tc_vblock comment): one wave
// owns one strip for the whole pass and a workgroup holds 4 strips (64
// columns), two workgroups per chain.  The strip lives in MFMA accumulators
// (8 C tiles of 16x16); in the chain k order those registers are directly the
// B operand of W h and, transposed by an identity product, the rows of the
// bf16 entry-state store.  W, U and K of chunk c+1 are fetched into registers
// while chunk c computes and staged in LDS between two barriers.
// Precision: h and uc stay float32 between chunks; every product that feeds
// the state splits its non-bf16 operands into hi+lo bf16 pairs (W and h: three
// products; the decayed uc: two, K is exact bf16).
#include "gdn_device.h"

namespace gdn {

constexpr int kWP = 132;  // W tile pitch (floats)
constexpr int kUP = 68;   // U tile pitch (floats)
constexpr int kCols = 64; // state columns per workgroup

// Byte offset of K^T[d][t] (t a multiple of 4) in the LDS tile: rows of 64
// tokens (128 B) in 16-byte granules, granule index XOR-swizzled with
// f(d) = (d ^ d>>3) & 7 so that both the transposing stores (16 rows 8 apart)
// and the fragment loads (16 consecutive rows) spread over all banks.
__device__ __forceinline__ int kt_off(int d, int t) {
  const int f = (d ^ (d >> 3)) & 7;
  return d * 128 + ((((t >> 3) ^ f) & 7) << 4) + ((t >> 2) & 1) * 8;
}

__global__ __launch_bounds__(kThreads) void chunk_delta_h(Params p) {
  const int cg = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Seq s = seq_of(p, i);
  if (!s.ok || s.nchunks == 0) return; // length 0: the state is left as it is
  const int kh = (h * p.nk) / p.nv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int col0 = cg * kCols;         // workgroup's first column
  const int colw = col0 + 16 * wave;   // this wave's strip
  float *hp = state_of(p, i, h);

  __shared__ __align__(16) float Wsh[kChunk * kWP];
  __shared__ __align__(16) float Ush[kChunk * kUP];
  __shared__ __align__(16) unsigned char Ksh[kDim * kChunk * 2];
  __shared__ float Gsh[kChunk];

  // state strip: H[m][ii] = h[16m + 4q + ii][colw + r16]
  f32x4 H[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) H[m][ii] = hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16];

  // ---- prefetch registers --------------------------------------------------
  f32x4 wreg[8], ureg[4];
  u32x4 kreg[4];
  float greg = 0.f;
  const int dg = tid & 15, tg = tid >> 4; // K transpose: 8 columns x 4 tokens
  auto fetch = [&](int c) {
    const int64_t sl = slot_of(p, s, h, c);
    const int n = min(kChunk, s.len - c * kChunk);
    const float *wsrc = p.w + sl * (kChunk * kDim);
    const float *usrc = p.u + sl * (kChunk * kDim) + col0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid + kThreads * j;
      wreg[j] = *reinterpret_cast<const f32x4 *>(wsrc + (idx >> 5) * kDim + 4 * (idx & 31));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + kThreads * j;
      ureg[j] = *reinterpret_cast<const f32x4 *>(usrc + (idx >> 4) * kDim + 4 * (idx & 15));
    }
    const int64_t row0 = s.tok0 + int64_t(c) * kChunk;
    const uint16_t *ksrc = p.k + row0 * p.qk_row + int64_t(kh) * kDim + 8 * dg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * tg + j;
      kreg[j] = (t < n) ? *reinterpret_cast<const u32x4 *>(ksrc + int64_t(t) * p.qk_row)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < kChunk) greg = p.gc[sl * kChunk + tid];
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid + kThreads * j;
      *reinterpret_cast<f32x4 *>(Wsh + (idx >> 5) * kWP + 4 * (idx & 31)) = wreg[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + kThreads * j;
      *reinterpret_cast<f32x4 *>(Ush + (idx >> 4) * kUP + 4 * (idx & 15)) = ureg[j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t x0 = (kreg[0][e >> 1] >> sh) & 0xFFFFu, x1 = (kreg[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t x2 = (kreg[2][e >> 1] >> sh) & 0xFFFFu, x3 = (kreg[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<u32x2 *>(Ksh + kt_off(8 * dg + e, 4 * tg)) = u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
    }
    if (tid < kChunk) Gsh[tid] = greg;
  };

  const bf16x8 C0 = ident_chain(lane, 0), C1 = ident_chain(lane, 1);

  fetch(0);
  stash();
  __syncthreads();

  for (int c = 0; c < s.nchunks; ++c) {
    const int n = min(kChunk, s.len - c * kChunk);
    const int64_t sl = slot_of(p, s, h, c);
    if (c + 1 < s.nchunks) fetch(c + 1);

    // h -> hi/lo bf16, chain order over dk (k block kb = rows 32kb .. 32kb+31)
    bf16x8 Hh[4], Hl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) chain_split(H[2 * kb], H[2 * kb + 1], Hh[kb], Hl[kb]);

    // entry state: bf16(h) transposed by identity products, stored [dk][dv]
    {
      uint16_t *sdst = p.s_entry + sl * (kDim * kDim) + colw + 4 * q4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 t0 = mfma(Hh[kb], C0, zero4());
        const f32x4 t1 = mfma(Hh[kb], C1, zero4());
        *reinterpret_cast<u32x2 *>(sdst + (32 * kb + r16) * kDim) = pack4_bf16(t0[0], t0[1], t0[2], t0[3]);
        *reinterpret_cast<u32x2 *>(sdst + (32 * kb + 16 + r16) * kDim) = pack4_bf16(t1[0], t1[1], t1[2], t1[3]);
      }
    }

    // uc = U - W h   (C tile mt: column colw + r16, rows t = 16mt + 4q .. +3)
    f32x4 D[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t = 16 * mt + r16;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(Wsh + t * kWP + 32 * kb + 4 * q4);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(Wsh + t * kWP + 32 * kb + 16 + 4 * q4);
        const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        bf16x8 wh, wl;
        split8(x, wh, wl);
        acc = mfma(wh, Hh[kb], acc);
        acc = mfma(wh, Hl[kb], acc);
        acc = mfma(wl, Hh[kb], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) D[mt][ii] = Ush[(16 * mt + 4 * q4 + ii) * kUP + 16 * wave + r16] - acc[ii];
    }

    // uc store, transposed: uc[slot][dv][t .. t+3]
    {
      uint16_t *udst = p.uc + sl * (kDim * kChunk) + (colw + r16) * kChunk + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<u32x2 *>(udst + 16 * mt) = pack4_bf16(D[mt][0], D[mt][1], D[mt][2], D[mt][3]);
    }

    // h <- exp(G_n) h + K^T diag(exp(G_n - G)) uc
    const float Gn = Gsh[n - 1];
    const float en = expf(Gn);
#pragma unroll
    for (int m = 0; m < 8; ++m) H[m] *= en;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) D[mt][ii] *= expf(Gn - Gsh[16 * mt + 4 * q4 + ii]);
    bf16x8 Dh[2], Dl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) chain_split(D[2 * kb], D[2 * kb + 1], Dh[kb], Dl[kb]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int d = 16 * m + r16;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(Ksh + kt_off(d, 32 * kb + 4 * q4));
        const u32x2 y = *reinterpret_cast<const u32x2 *>(Ksh + kt_off(d, 32 * kb + 16 + 4 * q4));
        const bf16x8 ka = join8(x, y);
        H[m] = mfma(ka, Dh[kb], H[m]);
        H[m] = mfma(ka, Dl[kb], H[m]);
      }
    }

    __syncthreads(); // every wave is done with chunk c's LDS tiles
    if (c + 1 < s.nchunks) {
      stash();
      __syncthreads();
    }
  }

#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) hp[(16 * m + 4 * q4 + ii) * kDim + colw + r16] = H[m][ii];
}

hipError_t launch_stage2(const Params &p, hipStream_t stream) {
  dim3 grid(kDim / kCols, p.nv, p.B);
  hipLaunchKernelGGL(chunk_delta_h, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
