// Stage 2: chunk_delta_h with the chunk output (chunk_fwd_o) fused in.
//
// Page "spark_model/layers/ops/ssm_gdn_a3.rs", doc comment of gdn_prefill_fla,
// stages 2 and 3: a serial pass over the chunks of each (sequence, v-head) that
// emits the per-chunk entry states, updates h_state in place, and forms each
// chunk's output.  Per chunk, with h the entry state (stored [dk][dv], float32)
// and T' the UT transform from stage 1:
//   S_entry[c] = bf16(h^T)                                  ([dv][dk])
//   uc         = U - W h = T' (V - diag(exp(G)) K h)
//   O          = diag(exp(G)) Q h + A uc,  A = tril_incl(exp(G_t - G_s) q_t.k_s)
//   h         <- exp(G_n) h + K^T diag(exp(G_n - G)) uc     (G_n: last token)
// Stage 3 of the page reads the entry state and uc back from memory; here both
// are still in registers when the output is formed, so neither uc nor a second
// read of the entry state ever reaches HBM.
//
// The dv columns of h evolve independently, so the state is split into
// 16-column strips (the page's DV-block split, tc_vblock comment).  A
// workgroup covers S strips of one chain (S = 1, 2 or 4, chosen so the grid
// fills the chip: few long chains get more workgroups each):
//   * waves 0..S-1 (compute): one strip each for the whole pass.  The strip
//     lives in MFMA accumulators; in the chain k order those registers are the
//     B operand of K h and Q h directly, and so are the C tiles of
//     R = V - e^G K h (for T' R) and of uc (for K^T uc and A uc): the
//     dependent chain never leaves registers;
//   * waves S..S+3 (loaders), two pairs; the pair that owns chunk c+1 stages
//     it into the free half of a double-buffered LDS stage, from registers it
//     filled two steps earlier, then fetches chunk c+3:
//       - wave 0 of the pair: Q and K as whole rows (1 KB per load), written
//         to LDS row tiles, and from the row fragments it reads back, the
//         causal decayed scores A on MFMA;
//       - wave 1 of the pair: the T' fragments, the decays, and V as whole
//         rows.
//     The compute waves read K^T and their V tiles out of the row tiles with
//     transposing LDS reads.
// One barrier per chunk.  Entry states leave as 16-byte pieces (dk order
// perm_dk).  Outputs are turned by an identity product into 8-byte pieces of
// token rows, gathered per chunk in an LDS tile, and stored by the idle
// loader pair as whole row segments of the workgroup's columns.
// Precision: h is float32 between chunks; h, R and the decayed uc are split
// into bf16 hi+lo for the products that feed the state (K is exact in bf16, T'
// arrives split), so every product keeps ~2^-17 relative error with bf16 MFMA
// and float32 accumulation.  The output uses bf16(h) and bf16(uc) -- the
// page's stage 3 reads both in bf16 -- with float32 accumulation.
//
// Workgroup order: all workgroups that read one k-head's rows (its r v-heads
// x column groups) get the same blockIdx.x % 8, so that on a round-robin XCD
// dispatch they share one XCD's L2.
#include "gdn_device.h"

namespace gdn {

// Q and K tiles are kept as rows: 64 rows of 16 pieces of 16 bytes, piece p of
// row t at slot 16t + (p ^ sig(t % 16)), sig swapping the two bit pairs of a
// 4-bit row index.  Without bank conflicts, 16 lanes then write a whole row,
// read a row fragment (16 rows, one piece each), or read with the transposing
// load a 4 x 4 block of 8-byte half pieces (rows t0..t0+3, pieces p0..p0+3,
// t0 and p0 multiples of 4).
__device__ __forceinline__ int row_slot(int t, int piece) {
  return 16 * t + (piece ^ (((t & 3) << 2) | ((t >> 2) & 3)));
}
// The V tile: 64 rows of (up to) 8 pieces, the workgroup's 64 columns; piece p
// of row t at slot 8t + (p ^ (2 * ((t >> 1) & 1))).
__device__ __forceinline__ int vrow_slot(int t, int piece) { return 8 * t + (piece ^ (2 * ((t >> 1) & 1))); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives, as element e, element i % 4 of the four 16-bit values that lane
// 4e + i / 4 of its group addresses.
__device__ __forceinline__ u32x2 read_tr(const void *lds_base, int byte_off) {
  const lds_s16x4 *a = (const lds_s16x4 *)((const __attribute__((address_space(3))) char *)lds_base + byte_off);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a));
}

struct Stage {
  u32x4 kr[64 * 16];          // K rows: row fragments for K h and the scores, K^T for K^T uc
  u32x4 qr[64 * 16];          // Q rows: row fragments for Q h and the scores
  u32x4 tp[2 * kTpFrags * 64]; // T' fragments: 6 hi, then 6 lo
  u32x4 af[kTpFrags * 64];    // scores A, A operand of A uc: fragment tri_frag(mt, kb)
  u32x4 vr[64 * 8];           // V rows, the workgroup's columns
  float dec[2 * kChunk];      // exp(G_t), exp(G_{n-1} - G_t)
};

// Split two C tiles (a k block of 32 rows, chain order) into hi / lo bf16
// fragments.  hi = bf16(x); x - hi is exact in float32 and comes from one bf16
// dot product per element, (hi0, hi1) . (-1, 0) + x0, with the constant pairs
// in registers m0, m1 (an inline constant would be read as the float32 -1.0).
__device__ __forceinline__ void split_tiles(const f32x4 &t0, const f32x4 &t1, uint32_t m0, uint32_t m1, bf16x8 &hi,
                                            bf16x8 &lo) {
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
__global__ __launch_bounds__((kStrips + 4) * 64) void chunk_delta_h_fwd_o(Params p) {
  constexpr int kGroups = 8 / kStrips; // workgroups per chain
  constexpr bool kAhead = kStrips < 4;  // compute waves read LDS operands a block ahead
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
  const int col0 = cg * 16 * kStrips; // first column of this workgroup

  __shared__ Stage st[2];
  // Output tiles of the last two chunks, [token][workgroup column] bf16 with a
  // row pitch of 32 * kStrips + 16 bytes (16 rows of one column block fall in
  // distinct banks).  A compute wave writes its strip of chunk c into tile
  // c % 2; during step c+1 the idle loader pair stores whole row segments of
  // it; tile c % 2 is next written in step c+2, after the barrier that ends
  // step c+1.
  constexpr int kOPitch = 32 * kStrips + 16;
  __shared__ __align__(16) char ost[2][kChunk * kOPitch];

  // =========================== loader waves ===============================
  if (wave >= kStrips) {
    // Loader li = wave - S is wave 0 of its pair (role 0) for li < 2.  With
    // waves dealt to the four SIMDs in turn, the two role-0 waves (the heavy
    // ones) then share no SIMD with a compute wave when S <= 2.
    const int pair = (wave - kStrips) & 1; // owns chunks c with c % 2 == pair
    const int role = (wave - kStrips) >> 1;
    const int nrow = lane >> 4, piece = lane & 15; // whole-row loads: 4 rows per instruction

    if (role == 0) {
      // ---- Q, K rows, and the scores from them --------------------------------
      u32x4 qx[16], kx[16]; // qx[j] = Q[4j + lane/16][8 (lane%16) .. +7]
      float gt[4];          // G at t = 16mt + r16
      f32x4 gs[4];          // G at s = 16ms + 4q .. +3
      auto fetch = [&](int c) {
        const int nn = min(kChunk, s.len - c * kChunk);
        // chunk bases are wave-uniform; a lane adds a 32-bit offset (row
        // pitches are bounded so that 64 rows stay below 2^31 bytes)
        const int64_t row0 = (s.tok0 + int64_t(c) * kChunk) * p.qk_row + int64_t(kh) * kDim;
        const char *qc = reinterpret_cast<const char *>(p.q + row0);
        const char *kc = reinterpret_cast<const char *>(p.k + row0);
        const uint32_t pitch = uint32_t(p.qk_row) * 2u;
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          // rows past the sequence end repeat its last row: they only reach
          // rows of products that are never stored, or meet zero rows of T'
          const uint32_t off = uint32_t(min(4 * jr + nrow, nn - 1)) * pitch + 16u * piece;
          qx[jr] = *reinterpret_cast<const u32x4 *>(qc + off);
          kx[jr] = *reinterpret_cast<const u32x4 *>(kc + off);
        }
        const float *gc = p.gc + slot_of(p, s, h, c) * kChunk;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          gt[m] = gc[16 * m + r16];
          gs[m] = *reinterpret_cast<const f32x4 *>(gc + 16 * m + 4 * q4);
        }
      };
      auto stash = [&](Stage &S) {
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          S.qr[row_slot(4 * jr + nrow, piece)] = qx[jr];
          S.kr[row_slot(4 * jr + nrow, piece)] = kx[jr];
        }
        // Row fragments are read back from the tiles this wave just wrote, a
        // few at a time: frag(T, mt, kb) = rows 16mt + r16, columns 32kb + 8q .. +7.
        auto frag = [&](const u32x4 *T, int mt, int kb) {
          return __builtin_bit_cast(bf16x8, T[row_slot(16 * mt + r16, 4 * kb + q4)]);
        };
        // C(ms, mt)[s][t] = q_t . k_s: A = K rows s, B = Q rows t; lane holds
        // column t = 16mt + r16, rows s = 16ms + 4q .. +3.  All Q fragments are
        // held; each K row tile is read once and used for every mt >= ms.
        bf16x8 qf[16];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) qf[4 * mt + kk] = frag(S.qr, mt, kk);
        f32x4 sc[4][4]; // sc[mt][ms], ms <= mt
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          bf16x8 kf[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kf[kk] = frag(S.kr, ms, kk);
#pragma unroll
          for (int mt = ms; mt < 4; ++mt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[kk], qf[4 * mt + kk], acc);
            sc[mt][ms] = acc;
          }
        }
        // masked to s <= t and decayed by exp(G_t - G_s), two vertically
        // stacked tiles are the chain-order A fragment (mt, kb) of A uc
        constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int t = 16 * mt + r16;
          const float g2t = gt[mt] * kLog2e;
#pragma unroll
          for (int ms = 0; ms <= mt; ++ms)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int si = 16 * ms + 4 * q4 + ii;
              sc[mt][ms][ii] = (si <= t) ? __builtin_amdgcn_exp2f(g2t - gs[ms][ii] * kLog2e) * sc[mt][ms][ii] : 0.f;
            }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (2 * kb > mt) continue;
            const f32x4 hi_tile = (2 * kb + 1 <= mt) ? sc[mt][2 * kb + 1] : zero4();
            S.af[tri_frag(mt, kb) * 64 + lane] = __builtin_bit_cast(u32x4, chain_frag(sc[mt][2 * kb], hi_tile));
          }
        }
      };
      if (pair < s.nchunks) fetch(pair);
      if (pair == 0) {
        stash(st[0]);
        if (2 < s.nchunks) fetch(2);
      }
      __syncthreads();
      for (int c = 0; c < s.nchunks; ++c) {
        if (((c + 1) & 1) == pair && c + 1 < s.nchunks) {
          stash(st[(c + 1) & 1]);
          if (c + 3 < s.nchunks) fetch(c + 3);
        }
        __syncthreads();
      }
      return;
    }

    // ---- T', decays, V rows --------------------------------------------------
    u32x4 tx[2 * kTpFrags];
    float d0 = 0.f, d1 = 0.f;
    // V rows of the workgroup's 16 * kStrips columns: 2 * kStrips pieces per row,
    // 32 / kStrips rows per load; vx[jj] = piece vpiece of row vrow0 + jj * vrows
    constexpr int kVPieces = 2 * kStrips, kVRows = 64 / kVPieces;
    const int vpiece = lane % kVPieces, vrow0 = lane / kVPieces;
    u32x4 vx[kVPieces];
    auto fetch = [&](int c) {
      const int64_t sl = slot_of(p, s, h, c);
      const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(p.tp + sl * (kTpBytes / 2));
#pragma unroll
      for (int f = 0; f < 2 * kTpFrags; ++f) tx[f] = tsrc[f * 64 + lane];
      d0 = p.dec[sl * 2 * kChunk + lane];
      d1 = p.dec[sl * 2 * kChunk + kChunk + lane];
      const int nn = min(kChunk, s.len - c * kChunk);
      const char *vc = reinterpret_cast<const char *>(p.v + (s.tok0 + int64_t(c) * kChunk) * p.v_row + int64_t(h) * kDim + col0);
      const uint32_t pitch = uint32_t(p.v_row) * 2u;
#pragma unroll
      for (int jj = 0; jj < kVPieces; ++jj) {
        const uint32_t off = uint32_t(min(vrow0 + jj * kVRows, nn - 1)) * pitch + 16u * vpiece;
        vx[jj] = *reinterpret_cast<const u32x4 *>(vc + off);
      }
    };
    auto stash = [&](Stage &S) {
#pragma unroll
      for (int f = 0; f < 2 * kTpFrags; ++f) S.tp[f * 64 + lane] = tx[f];
      S.dec[lane] = d0;
      S.dec[kChunk + lane] = d1;
#pragma unroll
      for (int jj = 0; jj < kVPieces; ++jj) S.vr[vrow_slot(vrow0 + jj * kVRows, vpiece)] = vx[jj];
    };
    // outputs of chunk co (staged in tile co % 2): whole row segments of the
    // workgroup's columns, 2 * kStrips pieces of 16 bytes per token row
    const int64_t orow = int64_t(p.nv) * kDim;
    auto store_out = [&](int co) {
      const int nn = min(kChunk, s.len - co * kChunk);
      char *oc = reinterpret_cast<char *>(p.out + (s.tok0 + int64_t(co) * kChunk) * orow + int64_t(h) * kDim + col0);
      const uint32_t opitch = uint32_t(orow) * 2u;
#pragma unroll
      for (int jj = 0; jj < kVPieces; ++jj) {
        const int t = vrow0 + jj * kVRows;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(&ost[co & 1][t * kOPitch + 16 * vpiece]);
        if (t < nn) *reinterpret_cast<u32x4 *>(oc + uint32_t(t) * opitch + 16u * vpiece) = val;
      }
    };
    if (pair < s.nchunks) fetch(pair);
    if (pair == 0) {
      stash(st[0]);
      if (2 < s.nchunks) fetch(2);
    }
    __syncthreads();
    for (int c = 0; c < s.nchunks; ++c) {
      if (((c + 1) & 1) == pair && c + 1 < s.nchunks) {
        stash(st[(c + 1) & 1]);
        if (c + 3 < s.nchunks) fetch(c + 3);
      }
      // the idle pair stores the previous chunk's outputs
      if ((c & 1) == pair && c >= 1) store_out(c - 1);
      __syncthreads();
    }
    if ((s.nchunks & 1) == pair) store_out(s.nchunks - 1);
    return;
  }

  // =========================== compute waves ==============================
  const int colw = col0 + 16 * wave; // this wave's strip
  float *hp = state_of(p, i, h);
  f32x4 H[8]; // H[m][ii] = h[perm_dk(16m + 4q + ii)][colw + r16]
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) H[m][ii] = hp[perm_dk(16 * m + 4 * q4 + ii) * kDim + colw + r16];

  // bf16 pairs (-1, 0) and (0, -1) for split_tiles, kept in registers
  uint32_t m0 = 0x0000BF80u, m1 = 0xBF800000u;
  asm volatile("" : "+v"(m0));
  asm volatile("" : "+v"(m1));
  const bf16x8 C0 = ident_chain(lane, 0), C1 = ident_chain(lane, 1);

  __syncthreads(); // chunk 0 staged

  for (int c = 0; c < s.nchunks; ++c) {
    const Stage &S = st[c & 1];
    const int64_t sl = slot_of(p, s, h, c);

    // h -> hi/lo bf16, chain order over dk (a lane's eight values are dk
    // 32kb + 8q .. +7); bf16(h) is also the entry state
    bf16x8 Hh[4], Hl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) split_tiles(H[2 * kb], H[2 * kb + 1], m0, m1, Hh[kb], Hl[kb]);
    {
      // S_c = h^T: row dv = colw + r16, dk = 32kb + 8q .. +7
      uint16_t *sdst = p.s_entry + sl * (kDim * kDim) + (colw + r16) * kDim + 8 * q4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<u32x4 *>(sdst + 32 * kb) = __builtin_bit_cast(u32x4, Hh[kb]);
    }

    // K h  (C tile mt: column colw + r16, rows t = 16mt + 4q .. +3); the row
    // fragments of block kb+1 are in flight while block kb's products issue
    auto kfrag = [&](const u32x4 *T, int mt, int kb) {
      return __builtin_bit_cast(bf16x8, T[row_slot(16 * mt + r16, 4 * kb + q4)]);
    };
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    {
      bf16x8 ka[2][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ka[0][mt] = kfrag(S.kr, mt, 0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < 3) {
          // with few compute waves per CU, read block kb+1 before block kb's
          // products (latency hidden); with four, read it after them (fewer
          // reads in flight at once on the shared LDS)
          if constexpr (kAhead) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ka[(kb + 1) & 1][mt] = kfrag(S.kr, mt, kb + 1);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(ka[kb & 1][mt], Hh[kb], acc[mt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma(ka[kb & 1][mt], Hl[kb], acc[mt]);
        if constexpr (!kAhead) {
          if (kb < 3) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ka[(kb + 1) & 1][mt] = kfrag(S.kr, mt, kb + 1);
          }
        }
      }
    }

    // R = V - diag(exp(G)) K h, split; the output's state term Q h (bf16 h)
    // is off the dependent chain and issues among R's vector instructions
    f32x4 eg[4];
    u32x2 vv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      eg[mt] = *reinterpret_cast<const f32x4 *>(S.dec + 16 * mt + 4 * q4);
      // V[16mt + 4q + ii][colw + r16], ii = 0..3: a transposing read of the V rows
      vv[mt] = read_tr(S.vr, vrow_slot(16 * mt + 4 * q4 + (r16 >> 2), 2 * wave + ((r16 & 3) >> 1)) * 16 + 8 * (r16 & 1));
    }
    bf16x8 qa[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) qa[4 * kb + mt] = kfrag(S.qr, mt, kb);
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t pr = vv[mt][ii >> 1];
        const float v = __builtin_bit_cast(float, (ii & 1) ? (pr & 0xFFFF0000u) : (pr << 16));
        R[mt][ii] = v - eg[mt][ii] * acc[mt][ii];
      }
    f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) O[mt] = mfma(qa[4 * kb + mt], Hh[kb], O[mt]);
    bf16x8 Rh[2], Rl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_tiles(R[2 * kb], R[2 * kb + 1], m0, m1, Rh[kb], Rl[kb]);
    if constexpr (kAhead) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); // then four VALU
      }
    }

    // uc = T' R  (T' is lower triangular: fragment (mt, 1) is zero for mt < 2);
    // all T' fragments are read up front
    bf16x8 th[kTpFrags], tl[kTpFrags];
    auto tpfrag = [&](int f) {
      th[f] = __builtin_bit_cast(bf16x8, S.tp[f * 64 + lane]);
      tl[f] = __builtin_bit_cast(bf16x8, S.tp[(kTpFrags + f) * 64 + lane]);
    };
    if constexpr (kAhead) {
#pragma unroll
      for (int f = 0; f < kTpFrags; ++f) tpfrag(f);
    }
    f32x4 D[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!kAhead) {
#pragma unroll
        for (int mt = 2 * kb; mt < 4; ++mt) tpfrag(tri_frag(mt, kb));
      }
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(th[tri_frag(mt, kb)], Rh[kb], D[mt]);
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(th[tri_frag(mt, kb)], Rl[kb], D[mt]);
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) D[mt] = mfma(tl[tri_frag(mt, kb)], Rh[kb], D[mt]);
    }
    bf16x8 af[kTpFrags];
    if constexpr (kAhead) {
#pragma unroll
      for (int f = 0; f < kTpFrags; ++f) af[f] = __builtin_bit_cast(bf16x8, S.af[f * 64 + lane]);
    }
    // K^T fragment (m, kb): row dk = perm_dk(16m + r16), tokens 32kb + chain
    // order -- two transposing reads of the K rows
    auto ktfrag = [&](int m, int kb) {
      const int pc = 4 * (m >> 1) + (r16 & 3), hb = 8 * (m & 1);
      const int t0 = 32 * kb + 4 * q4 + (r16 >> 2);
      const u32x2 lo = read_tr(S.kr, row_slot(t0, pc) * 16 + hb);
      const u32x2 hi = read_tr(S.kr, row_slot(t0 + 16, pc) * 16 + hb);
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    bf16x8 ka[2][8];
    if constexpr (kAhead) {
#pragma unroll
      for (int m = 0; m < 8; ++m) ka[0][m] = ktfrag(m, 0);
    }

    // h <- exp(G_n) h + K^T diag(exp(G_n - G)) uc; the output's intra-chunk
    // term A bf16(uc) issues among the vector instructions of the split
    const float en = S.dec[kChunk - 1]; // exp(G) of the last row = exp(G_n): rows past the end repeat it
    bf16x8 ub[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ub[kb] = chain_frag(D[2 * kb], D[2 * kb + 1]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) O[mt] *= eg[mt];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) {
        if constexpr (!kAhead) af[tri_frag(mt, kb)] = __builtin_bit_cast(bf16x8, S.af[tri_frag(mt, kb) * 64 + lane]);
        O[mt] = mfma(af[tri_frag(mt, kb)], ub[kb], O[mt]);
      }
#pragma unroll
    for (int m = 0; m < 8; ++m) H[m] *= en;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) D[mt] *= *reinterpret_cast<const f32x4 *>(S.dec + kChunk + 16 * mt + 4 * q4);
    bf16x8 Dh[2], Dl[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) split_tiles(D[2 * kb], D[2 * kb + 1], m0, m1, Dh[kb], Dl[kb]);
    if constexpr (kAhead) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1); // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 1); // then six VALU
      }
    }
    if constexpr (!kAhead) {
#pragma unroll
      for (int m = 0; m < 8; ++m) ka[0][m] = ktfrag(m, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (kAhead) {
        if (kb == 0) {
#pragma unroll
          for (int m = 0; m < 8; ++m) ka[1][m] = ktfrag(m, 1);
        }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) H[m] = mfma(ka[kb][m], Dh[kb], H[m]);
#pragma unroll
      for (int m = 0; m < 8; ++m) H[m] = mfma(ka[kb][m], Dl[kb], H[m]);
      if constexpr (!kAhead) {
        if (kb == 0) {
#pragma unroll
          for (int m = 0; m < 8; ++m) ka[1][m] = ktfrag(m, 1);
        }
      }
    }

    // output: bf16, turned by an identity product so a lane holds 4
    // consecutive columns of one token, into this chunk's output tile
    {
      char *ot = &ost[c & 1][32 * wave + 8 * q4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 oa = chain_frag(O[2 * kk], O[2 * kk + 1]);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f32x4 d = mfma(oa, hf ? C1 : C0, zero4());
          const int t = 32 * kk + 16 * hf + r16;
          *reinterpret_cast<u32x2 *>(ot + t * kOPitch) = pack4_bf16(d[0], d[1], d[2], d[3]);
        }
      }
    }

    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) hp[perm_dk(16 * m + 4 * q4 + ii) * kDim + colw + r16] = H[m][ii];
}

namespace {
int compute_units() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <int kStrips>
hipError_t launch_with(const Params &p, hipStream_t stream) {
  const int r = p.nv / p.nk;
  const int kgroups = p.B * p.nk;
  const int blocks = 8 * ((kgroups + 7) / 8) * r * (8 / kStrips);
  hipLaunchKernelGGL(chunk_delta_h_fwd_o<kStrips>, dim3(blocks), dim3((kStrips + 4) * 64), 0, stream, p);
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
