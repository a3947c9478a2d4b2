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
//     B operand of K h (and of Q h), and so are the C tiles of
//     R = V - e^G K h (for T' R) and of uc (for K^T uc and A uc): the
//     dependent chain never leaves registers.  Step c runs chunk c's chain;
//     with S = 4 it also forms the state term diag(exp(G)) Q h and finishes
//     chunk c-1's output with A uc, whose scores were formed during step c-1;
//   * the loader waves, in two pairs that take turns.  In step c the active
//     pair of each role stages chunk c+1 into the free half of a
//     double-buffered LDS stage, from registers it filled two steps earlier,
//     then fetches chunk c+3; the idle pair works on chunk c, already staged.
//     With S = 4 (four loaders): role 0 fetches the Q rows and K rows 0..31
//     (1 KB per load) and stores the output tile of chunk c-2; role 1 fetches
//     K rows 32..63, the T' fragments (bf16 hi + lo), the gate sums G (from
//     which it forms the decays as it stages them; with q/k normalisation the
//     row scales too) and V rows; the idle waves of both roles form the causal
//     decayed scores A of chunk c on MFMA, half each, for the compute waves.
//     (All K rows on role 0, that wave's loads were the longest part of its
//     step, and the ragged workload's spine ran 7 % slower; all on role 1,
//     the batched workload's ran 2 % slower.)
//     With S <= 2 (six loaders; two SIMDs hold no compute wave): role 1 on
//     those SIMDs fetches T', G and V as above; its idle wave forms chunk c's
//     scores and keeps them, and in step c+1 forms chunk c's output from the
//     compute waves' bf16 h and bf16 uc, left in LDS; role 0 fetches the Q
//     rows and stores the output tiles, role 2 the K rows.  After each
//     barrier the Q- and K-row loaders wait before staging, so that the
//     compute waves' first LDS reads of the step go first.
//     The compute waves read K^T and their V tiles out of the row tiles with
//     transposing LDS reads.
// One barrier per chunk (and one after the last).  Entry states (when asked
// for) leave as 16-byte pieces of [dv][dk] rows, straight from the bf16 h
// fragments (dk order perm_dk).  The output is formed transposed, so a
// lane holds 8-byte pieces of token rows; they are gathered per chunk in an
// LDS tile and stored by a loader as whole row segments of the workgroup's
// columns.
// Every double-buffered region (stage, scores, h and uc tiles, output tile) is
// written in one step and read in the next, and written again only after the barrier that
// ends the reading step.
// Precision: h is float32 between chunks; h, R and the decayed uc are split
// into bf16 hi+lo for the products that feed the state (K is exact in bf16;
// T' arrives as a bf16 hi + lo pair), so every product keeps ~2^-17
// relative error with bf16 MFMA and float32 accumulation.  The output uses bf16(h) and bf16(uc) -- the
// page's stage 3 reads both in bf16 -- with float32 accumulation.
//
// Workgroup order: all workgroups that read one k-head's rows (its r v-heads
// x column groups) get the same blockIdx.x % 8, so that on a round-robin XCD
// dispatch they share one XCD's L2.
#include "gdn_device.h"

namespace gdn {

// Q and K tiles are kept as rows: 64 rows of 16 pieces of 16 bytes, piece p of
// row t at slot 16t + (p ^ swz(t % 16)), swz moving the bits (t0, t1, t2, t3)
// of the row index to bits (0, 2, 3, 1).  gfx950's LDS serves a 16-byte read
// in four passes of 16 lanes, lanes 0..31 split by the parity of bits 2..4 of
// the lane id (likewise 32..63), and a pass is free of bank conflicts when
// its 16 lanes touch 16 distinct 16-byte columns of the 256-byte bank row;
// 8-byte reads take passes of 32 consecutive lanes, 16-byte writes passes of
// 8 consecutive lanes over 128 bytes.  With swz, 16 lanes write a whole row,
// and a row fragment (16 rows, one piece each) is read, without conflicts;
// the transposing read of a 4 x 4 block of 8-byte half pieces (rows t0..t0+3,
// pieces p0..p0+3, t0 and p0 multiples of 4) meets each bank twice (its 32
// lanes read one half of each piece).
__device__ __forceinline__ int row_slot(int t, int piece) {
  const int swz = (t & 1) | ((t & 2) << 1) | ((t & 4) << 1) | ((t & 8) >> 2);
  return 16 * t + (piece ^ swz);
}
// The V tile: 64 rows of (up to) 8 pieces, the workgroup's columns; piece p of
// row t at slot 8t + (p ^ vswz(t)), vswz(t) = 2 ((t / 2) % 4) ^ 4 (t % 2): the
// transposing read of 8 rows x 2 pieces and the row writes (8 lanes over 1,
// 2 or 4 rows) meet each bank once.
__device__ __forceinline__ int vrow_slot(int t, int piece) { return 8 * t + (piece ^ ((2 * ((t >> 1) & 3)) ^ (4 * (t & 1)))); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives, as element e, element i % 4 of the four 16-bit values that lane
// 4e + i / 4 of its group addresses.
__device__ __forceinline__ u32x2 read_tr(const void *lds_base, int byte_off) {
  const lds_s16x4 *a = (const lds_s16x4 *)((const __attribute__((address_space(3))) char *)lds_base + byte_off);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a));
}

// Section stamps (profiling build only): every wave reads the shader clock
// (s_memtime) at its section marks into registers, and the 100 MHz clock
// (s_memrealtime) once per step; after the step's barrier, lane 0 of each wave
// of workgroup 0 stores the marks of steps kStampFirst.. (one row of
// kStampSlots per step, mark 15 the 100 MHz stamp).  The marks add no branch
// and no wait inside a step: the results are first used by the store after
// the barrier.  In the product build the marks are empty.
#ifdef GDN_SECTION_STAMPS
#define GDN_STAMP_DECL unsigned long long ts_[kStampSlots] = {}
#define GDN_STAMP(id) (ts_[id] = __builtin_amdgcn_s_memtime())
#define GDN_RSTAMP() (ts_[15] = __builtin_amdgcn_s_memrealtime())
#define GDN_STAMP_FLUSH(c)                                                                                            \
  do {                                                                                                                \
    if (p.stamps && blockIdx.x == 0 && lane == 0 && (c) >= kStampFirst && (c) < kStampFirst + kStampSteps) {         \
      _Pragma("unroll") for (int id_ = 0; id_ < kStampSlots; ++id_)                                                  \
          p.stamps[(size_t(wave) * kStampSteps + ((c) - kStampFirst)) * kStampSlots + id_] = ts_[id_];               \
    }                                                                                                                 \
  } while (0)
#else
#define GDN_STAMP_DECL
#define GDN_STAMP(id) ((void)0)
#define GDN_RSTAMP() ((void)0)
#define GDN_STAMP_FLUSH(c) ((void)0)
#endif

template <int N> struct Mask {
  static constexpr int value = N;
};

// The per-token factors of a chunk, formed by the role-1 loader from G (and,
// with q/k normalisation, the row scales sk = 1/|k_t|, sq = 1/|q_t|; without
// it both are 1): the normalised keys and queries are diag(sk) K and
// diag(sq) Q, so every product keeps the exact bf16 rows and the scales ride
// on factors that are applied anyway.
struct Stage {
  u32x4 kr[64 * 16];          // K rows: row fragments for K h and the scores, K^T for K^T uc
  u32x4 qr[64 * 16];          // Q rows: row fragments for Q h and the scores
  u32x4 tp[2 * kTpFrags * 64]; // T' fragments: 6 hi, then 6 lo
  u32x4 vr[64 * 8];           // V rows, the workgroup's columns
  float eg[kChunk];           // exp(G_t) sk_t:       R = V - diag(eg) (K h)
  float dn[kChunk];           // exp(G_n - G_t) sk_t: h += K^T diag(dn) uc
  float dq[kChunk];           // exp(G_t) sq_t:       O = diag(dq) (Q h) + A uc
  float g2q[kChunk];          // log2(e) G_t + log2(sq_t) \ A[t][s] = exp2(g2q_t - g2k_s) q_t.k_s
  float g2k[kChunk];          // log2(e) G_s - log2(sk_s) /
  float en[4];                // en[0] = exp(G_n), G_n the gate sum at the last token
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

// Loader waves per workgroup: four, and six where the output moves onto the
// loaders (S <= 2, below).
template <int kStrips> constexpr int loader_waves() { return kStrips <= 2 ? 6 : 4; }

// With S <= 2, after each barrier the Q-row loaders (which share a SIMD with
// the compute waves) and the K-row loaders sleep before they stage, in units
// of 64 cycles, so that the compute waves' first LDS reads and instructions of
// the step are not queued behind the stage writes; the staging still ends
// well before the step does.  Measured on MI355X at one and two strips: the
// spine's step falls by 13% (T = 65536, 48 chains) and 7% (T = 4096, one
// chain) against no delay; the time is flat for Q-row delays of 16..24 and
// K-row delays of 8..12, and any delay of the score/output loaders costs time.
constexpr int kQRowDelay = 20, kKRowDelay = 10;

template <int kStrips, bool kEntry>
__global__ __launch_bounds__((kStrips + loader_waves<kStrips>()) * 64) void chunk_delta_h_fwd_o(Params p) {
  // With S <= 2 strips per workgroup two SIMDs hold no compute wave and the
  // LDS has room, so the output moves off the compute waves (kOL): the loader
  // that formed chunk c's scores in step c keeps them, chunk c's Q fragments
  // and its output decays in registers, and in step c+1 reads the compute
  // waves' bf16 h and bf16 uc of chunk c from LDS (tiles ht, ut, written in
  // step c) and forms O^T = diag(exp(G)) (h^T Q^T) + uc^T A^T itself.  The Q
  // and K rows are then fetched by two waves per pair instead of one.
  constexpr bool kOL = kStrips <= 2;
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
  const int nch = s.nchunks;

  // the wave index is made scalar, so that branches on a wave's role are
  // scalar branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, r16 = lane & 15;
  const int col0 = cg * 16 * kStrips; // first column of this workgroup

  __shared__ Stage st[2];
  // scores A of chunk c (A operand of A uc, fragment tri_frag(mt, kb)) in
  // afb[c % 2]: formed in step c, used in step c+1 (S = 4; with kOL they stay
  // in the registers of the loader that formed them)
  __shared__ u32x4 afb[2][kOL ? 1 : kTpFrags * 64];
  // kOL: bf16 h and bf16 uc of chunk c per compute wave, its fragments Hh[kb]
  // and ub[kb] as 64 lanes x 16 bytes each, in ht / ut [c % 2][wave]: written
  // in step c, read in step c+1, written again in step c+2
  __shared__ u32x4 ht[kOL ? 2 * kStrips * 4 * 64 : 1];
  __shared__ u32x4 ut[kOL ? 2 * kStrips * 2 * 64 : 1];
  // Output tiles, [token][workgroup column] bf16 with a row pitch of
  // 32 * kStrips + 16 bytes (16 rows of one column block fall in distinct
  // banks): chunk c's tile ost[c % 2] is written in step c+1 and stored in
  // step c+2.
  constexpr int kOPitch = 32 * kStrips + 16;
  __shared__ __align__(16) char ost[2][kChunk * kOPitch];

  // =========================== loader waves ===============================
  if (wave >= kStrips) {
    // Loader li = wave - S belongs to pair li % 2.  Waves are dealt to the four
    // SIMDs in turn, so for S <= 2 loaders li = 0, 1 sit on SIMDs without a
    // compute wave: they take role 1 (T', V, gate sums; the score products and,
    // with kOL, the output; half the K rows for S = 4); role 0 (Q rows, and
    // half the K rows for S = 4; the output stores) shares a SIMD with a
    // compute wave; with kOL role 2 (the K rows) sits beside a role-1 wave.  For S = 4 every SIMD holds one compute wave
    // and one loader.
    const int li = wave - kStrips;
    const int pair = li & 1; // stages chunks c with c % 2 == pair
    const int role = kOL ? ((li >> 1) == 0 ? 1 : (li >> 1) == 1 ? 0 : 2) : (li >> 1);
    const int nrow = lane >> 4, piece = lane & 15; // whole-row loads: 4 rows per instruction
    // rows of the workgroup's 16 * kStrips columns: 2 * kStrips pieces per row
    constexpr int kVPieces = 2 * kStrips, kVRows = 64 / kVPieces;
    const int vpiece = lane % kVPieces, vrow0 = lane / kVPieces;

    // scores of the chunk staged in S, into A: C(ms, mt)[s][t] = q_t . k_s
    // (A = K rows s, B = Q rows t; lane holds column t = 16mt + r16, rows
    // s = 16ms + 4q .. +3), masked to s <= t and decayed by exp(G_t - G_s)
    // (times sq_t sk_s with q/k normalisation);
    // two vertically stacked tiles are the chain-order A fragment (mt, kb),
    // left in A[tri_frag(mt, kb)]; the Q row fragments are left in qf.
    // Only the fragments of the row blocks mt in the bit mask are formed (the
    // caller passes Mask<bits>).
    auto scores = [&](const Stage &S, u32x4 (&A)[kTpFrags], bf16x8 (&qf)[16], auto mask_tag)
                      __attribute__((always_inline)) {
      constexpr int mask = decltype(mask_tag)::value;
      constexpr int top = (mask & 8) ? 3 : (mask & 4) ? 2 : (mask & 2) ? 1 : 0;
      auto frag = [&](const u32x4 *T, int mt, int kb) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, T[row_slot(16 * mt + r16, 4 * kb + q4)]);
      };
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          if (mask & (1 << mt)) qf[4 * mt + kk] = frag(S.qr, mt, kk);
      f32x4 sc[4][4]; // sc[mt][ms], ms <= mt
#pragma unroll
      for (int ms = 0; ms <= top; ++ms) {
        bf16x8 kf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[kk] = frag(S.kr, ms, kk);
#pragma unroll
        for (int mt = ms; mt < 4; ++mt) {
          if (!(mask & (1 << mt))) continue;
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[kk], qf[4 * mt + kk], acc);
          sc[mt][ms] = acc;
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (!(mask & (1 << mt))) continue;
        const int t = 16 * mt + r16;
        const float g2t = S.g2q[t];
#pragma unroll
        for (int ms = 0; ms <= mt; ++ms) {
          const f32x4 g2s = *reinterpret_cast<const f32x4 *>(S.g2k + 16 * ms + 4 * q4);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int si = 16 * ms + 4 * q4 + ii;
            sc[mt][ms][ii] = (si <= t) ? __builtin_amdgcn_exp2f(g2t - g2s[ii]) * sc[mt][ms][ii] : 0.f;
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (2 * kb > mt) continue;
          const f32x4 hi_tile = (2 * kb + 1 <= mt) ? sc[mt][2 * kb + 1] : zero4();
          A[tri_frag(mt, kb)] = __builtin_bit_cast(u32x4, chain_frag(sc[mt][2 * kb], hi_tile));
        }
      }
    };
    // S = 4: the fragments of the row blocks in the mask go to afb for the
    // compute waves
    auto scores_to_lds = [&](const Stage &S, u32x4 *dst, auto mask_tag) __attribute__((always_inline)) {
      constexpr int mask = decltype(mask_tag)::value;
      u32x4 A[kTpFrags];
      bf16x8 qf[16];
      scores(S, A, qf, mask_tag);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if ((mask & (1 << mt)) && 2 * kb <= mt) dst[tri_frag(mt, kb) * 64 + lane] = A[tri_frag(mt, kb)];
    };
    // S = 4: the Q or K rows 4 j0 .. 4 j1 - 1 of chunk c (the k-head's 256
    // bytes of each token row), rx[j] = row 4j + lane/16, bf16 8 (lane%16)
    // .. +7, and their place in a row tile of the stage
    auto fetch_rows = [&](const uint16_t *base, int c, u32x4 (&rx)[16], int j0, int j1) __attribute__((always_inline)) {
      const int nn = min(kChunk, s.len - c * kChunk);
      // chunk bases are wave-uniform; a lane adds a 32-bit offset (row
      // pitches are bounded so that 64 rows stay below 2^31 bytes)
      const char *src =
          reinterpret_cast<const char *>(base + (s.tok0 + int64_t(c) * kChunk) * p.qk_row + int64_t(kh) * kDim);
      const uint32_t pitch = uint32_t(p.qk_row) * 2u;
#pragma unroll
      for (int jr = 0; jr < 16; ++jr) {
        if (jr < j0 || jr >= j1) continue;
        // rows past the sequence end repeat its last row: they only reach
        // rows of products that are never stored, or meet zero rows of T'
        const uint32_t off = uint32_t(min(4 * jr + nrow, nn - 1)) * pitch + 16u * piece;
        rx[jr] = *reinterpret_cast<const u32x4 *>(src + off);
      }
    };
    auto stash_rows = [&](u32x4 *tile, const u32x4 (&rx)[16], int j0, int j1) __attribute__((always_inline)) {
#pragma unroll
      for (int jr = 0; jr < 16; ++jr)
        if (jr >= j0 && jr < j1) tile[row_slot(4 * jr + nrow, piece)] = rx[jr];
    };
    GDN_STAMP_DECL;
    if (role != 1) {
      // ---- Q rows (K rows with kOL role 2); outputs -----------------------
      // with kOL roles 0 and 2 move one operand each (Q rows, K rows) through
      // the same registers, chosen by a wave-uniform pointer rather than a
      // branch per load (a load under a branch waits for every load before it)
      constexpr int kOps = 1;
      const bool doQ = !kOL || role == 0;
      u32x4 rx[kOps][16]; // rx[o][j] = operand row 4j + lane/16, bf16 8 (lane%16) .. +7
      u32x4 kx[16];       // S = 4: K rows 0..31
      // At S = 4 (the Q rows and K rows 0..31) through the row helpers; with
      // kOL through the form below.  Both issue the same loads and stores, but the compiler
      // schedules each kernel's address arithmetic differently, and these are
      // the pairings measured fastest (the other way round: 2 % slower at
      // S <= 2, 3 % on the ragged workload at S = 4).
      auto fetch = [&](int c) __attribute__((always_inline)) {
        if constexpr (!kOL) {
          fetch_rows(p.q, c, rx[0], 0, 16);
          fetch_rows(p.k, c, kx, 0, 8);
          return;
        }
        const int nn = min(kChunk, s.len - c * kChunk);
        // chunk bases are wave-uniform; a lane adds a 32-bit offset (row
        // pitches are bounded so that 64 rows stay below 2^31 bytes)
        const int64_t row0 = (s.tok0 + int64_t(c) * kChunk) * p.qk_row + int64_t(kh) * kDim;
        const char *src[2] = {reinterpret_cast<const char *>((doQ ? p.q : p.k) + row0),
                              reinterpret_cast<const char *>(p.k + row0)};
        const uint32_t pitch = uint32_t(p.qk_row) * 2u;
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          // rows past the sequence end repeat its last row: they only reach
          // rows of products that are never stored, or meet zero rows of T'
          const uint32_t off = uint32_t(min(4 * jr + nrow, nn - 1)) * pitch + 16u * piece;
#pragma unroll
          for (int o = 0; o < kOps; ++o) rx[o][jr] = *reinterpret_cast<const u32x4 *>(src[o] + off);
        }
      };
      auto stash = [&](Stage &S) __attribute__((always_inline)) {
        if constexpr (!kOL) {
          stash_rows(S.qr, rx[0], 0, 16);
          stash_rows(S.kr, kx, 0, 8);
          return;
        }
        u32x4 *dst[2] = {doQ ? S.qr : S.kr, S.kr};
#pragma unroll
        for (int jr = 0; jr < 16; ++jr)
#pragma unroll
          for (int o = 0; o < kOps; ++o) dst[o][row_slot(4 * jr + nrow, piece)] = rx[o][jr];
      };
      // outputs of chunk co (tile co % 2): whole row segments of the
      // workgroup's columns
      const int64_t orow = int64_t(p.nv) * kDim;
      auto store_out = [&](int co) __attribute__((always_inline)) {
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
      if (pair < nch) fetch(pair);
      if (pair == 0) {
        stash(st[0]);
        if (2 < nch) fetch(2);
      }
      __syncthreads();
      for (int c = 0; c <= nch; ++c) {
        GDN_STAMP(0);
        if constexpr (kOL) {
          if (doQ)
            __builtin_amdgcn_s_sleep(kQRowDelay);
          else
            __builtin_amdgcn_s_sleep(kKRowDelay);
        }
        if (((c + 1) & 1) == pair && c + 1 < nch) {
          stash(st[(c + 1) & 1]);
          GDN_STAMP(1);
          if (c + 3 < nch) fetch(c + 3);
          GDN_STAMP(2);
        }
        // the idle pair stores the output of chunk c-2 and, for S = 4, forms
        // half of chunk c's scores
        if (doQ && (c & 1) == pair && c >= 2) store_out(c - 2);
        if constexpr (kStrips == 4)
          if ((c & 1) == pair && c < nch) scores_to_lds(st[c & 1], afb[c & 1], Mask<0x9>());
        GDN_STAMP(3);
        __syncthreads();
        GDN_STAMP(4);
        GDN_STAMP_FLUSH(c);
      }
      // after the last barrier: the last chunk's output
      if (doQ && (nch & 1) == pair) store_out(nch - 1);
      return;
    }

    // ---- T', gate sums (and row scales), V rows; scores ---------------------
    const bool norm = (p.opts & kOptNorm) != 0;
    u32x4 tx[2 * kTpFrags];  // T' as fetched and staged: bf16 hi (f), lo (6 + f)
    float gg = 0.f, skv = 1.f, sqv = 1.f;
    u32x4 vx[kVPieces];
    u32x4 kx[16]; // S = 4: K rows 32..63
    auto fetch = [&](int c) __attribute__((always_inline)) {
      const int64_t sl = slot_of(p, s, h, c);
      if constexpr (!kOL) fetch_rows(p.k, c, kx, 8, 16);
      const char *tsrc = reinterpret_cast<const char *>(p.tp) + sl * kTpBytes;
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int f = 0; f < kTpFrags; ++f) {
          const char *src = tsrc + part * kTpHalfBytes + tp_offset(f);
          if (tp_half(f)) { // the zero half above the diagonal is not stored
            const u32x2 x = *reinterpret_cast<const u32x2 *>(src + 8 * lane);
            tx[part * kTpFrags + f] = u32x4{x[0], x[1], 0u, 0u};
          } else {
            tx[part * kTpFrags + f] = *reinterpret_cast<const u32x4 *>(src + 16 * lane);
          }
        }
      gg = p.gc[sl * kChunk + lane];
      if (norm) {
        skv = p.nrm[sl * 2 * kChunk + lane];
        sqv = p.nrm[sl * 2 * kChunk + kChunk + lane];
      }
      const int nn = min(kChunk, s.len - c * kChunk);
      const char *vc = reinterpret_cast<const char *>(p.v + (s.tok0 + int64_t(c) * kChunk) * p.v_row + int64_t(h) * kDim + col0);
      const uint32_t pitch = uint32_t(p.v_row) * 2u;
#pragma unroll
      for (int jj = 0; jj < kVPieces; ++jj) {
        const uint32_t off = uint32_t(min(vrow0 + jj * kVRows, nn - 1)) * pitch + 16u * vpiece;
        vx[jj] = *reinterpret_cast<const u32x4 *>(vc + off);
      }
    };
    // the chunk's per-token factors from G (rows past the sequence end repeat
    // the last G, so lane 63 holds G_n)
    auto stash = [&](Stage &S) __attribute__((always_inline)) {
      if constexpr (!kOL) stash_rows(S.kr, kx, 8, 16);
#pragma unroll
      for (int f = 0; f < 2 * kTpFrags; ++f) S.tp[f * 64 + lane] = tx[f];
      const float Gn = __shfl(gg, kChunk - 1, 64);
      const float e = expf(gg), en = expf(Gn - gg);
      const float g2 = gg * 1.4426950408889634f; // log2(e) G
      S.eg[lane] = e * skv;
      S.dn[lane] = en * skv;
      S.dq[lane] = e * sqv;
      S.g2q[lane] = norm ? g2 + log2f(sqv) : g2;
      S.g2k[lane] = norm ? g2 - log2f(skv) : g2;
      if (lane == kChunk - 1) S.en[0] = e;
#pragma unroll
      for (int jj = 0; jj < kVPieces; ++jj) S.vr[vrow_slot(vrow0 + jj * kVRows, vpiece)] = vx[jj];
    };
    // kOL: chunk co's scores, Q fragments and output decays, kept from the
    // step that formed the scores (co) to the next, which forms its output
    u32x4 a_keep[kTpFrags];
    bf16x8 q_keep[16];
    float dq_keep[4];
    // kOL: the output of chunk co for the workgroup's strips, into its output
    // tile ost[co % 2]: O^T = diag(dq) (h^T Q^T) + uc^T A^T per strip, with
    // bf16 h and bf16 uc read from ht / ut
    auto output = [&](int co) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < kStrips; ++w) {
        const u32x4 *hti = ht + ((co & 1) * kStrips + w) * 4 * 64 + lane;
        const u32x4 *uti = ut + ((co & 1) * kStrips + w) * 2 * 64 + lane;
        f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 hb = __builtin_bit_cast(bf16x8, hti[kb * 64]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) O[mt] = mfma(hb, q_keep[4 * mt + kb], O[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) O[mt] *= dq_keep[mt];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ub = __builtin_bit_cast(bf16x8, uti[kb * 64]);
#pragma unroll
          for (int mt = 2 * kb; mt < 4; ++mt)
            O[mt] = mfma(ub, __builtin_bit_cast(bf16x8, a_keep[tri_frag(mt, kb)]), O[mt]);
        }
        char *ot = &ost[co & 1][32 * w + 8 * q4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          *reinterpret_cast<u32x2 *>(ot + (16 * mt + r16) * kOPitch) =
              pack4_bf16(O[mt][0], O[mt][1], O[mt][2], O[mt][3]);
      }
    };
    if (pair < nch) fetch(pair);
    if (pair == 0) {
      stash(st[0]);
      if (2 < nch) fetch(2);
    }
    __syncthreads();
    for (int c = 0; c <= nch; ++c) {
      GDN_STAMP(0);
      // the active pair stages chunk c+1, fetched two steps earlier
      if (((c + 1) & 1) == pair && c + 1 < nch) {
        stash(st[(c + 1) & 1]);
        GDN_STAMP(1);
        if (c + 3 < nch) fetch(c + 3);
        GDN_STAMP(2);
      }
      if constexpr (kOL) {
        // the active pair forms the output of chunk c-1, whose scores it
        // formed in step c-1; the idle pair forms (and keeps) chunk c's
        if (((c + 1) & 1) == pair && c >= 1) output(c - 1);
        if ((c & 1) == pair && c < nch) {
          scores(st[c & 1], a_keep, q_keep, Mask<0xF>());
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) dq_keep[mt] = st[c & 1].dq[16 * mt + r16];
        }
      } else {
        // the idle pair forms the scores of chunk c (with role 0 for S = 4)
        if ((c & 1) == pair && c < nch) scores_to_lds(st[c & 1], afb[c & 1], Mask<0x6>());
      }
      GDN_STAMP(3);
      __syncthreads();
      GDN_STAMP(4);
      GDN_STAMP_FLUSH(c);
    }
    return;
  }

  // =========================== compute waves ==============================
  GDN_STAMP_DECL;
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

  // LDS operand readers: row fragments of the Q / K tiles (rows 16mt + r16,
  // columns 32kb + 8q .. +7) and K^T fragments (rows dk = perm_dk(16m + r16),
  // tokens 32kb + chain order: two transposing reads of the K rows)
  auto rfrag = [&](const u32x4 *T, int mt, int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, T[row_slot(16 * mt + r16, 4 * kb + q4)]);
  };
  auto ktfrag = [&](const Stage &S, int m, int kb) __attribute__((always_inline)) {
    const int pc = 4 * (m >> 1) + (r16 & 3), hb = 8 * (m & 1);
    const int t0 = 32 * kb + 4 * q4 + (r16 >> 2);
    const u32x2 lo = read_tr(S.kr, row_slot(t0, pc) * 16 + hb);
    const u32x2 hi = read_tr(S.kr, row_slot(t0 + 16, pc) * 16 + hb);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  // interleave, in the current scheduling region, n MFMAs each followed by v
  // vector instructions
#define GDN_INTERLEAVE(n, v, id)                                                                                       \
  do {                                                                                                                 \
    _Pragma("unroll") for (int i_ = 0; i_ < (n); ++i_) {                                                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, id);                                                              \
      __builtin_amdgcn_sched_group_barrier(0x002, v, id);                                                              \
    }                                                                                                                  \
  } while (0)

  // The output is formed transposed, O^T = h^T Q^T + uc^T A^T, so that tile mt
  // holds, in lane (q, r), token 16mt + r and the four columns colw + 4q .. +3:
  // the split of h (chain order over dk) is the A operand of h^T Q^T as it is
  // the B operand of K h, and likewise bf16(uc) for uc^T A^T; the Q and score
  // fragments serve as B operands unchanged.
  f32x4 O[4];      // O^T of the chunk whose output is pending: diag(exp(G)) Q h so far
  bf16x8 ub[2];    // its bf16(uc), chain order over tokens
  // chunk c-1's output, finished in step c from the score fragments af: O^T +=
  // uc^T A^T, then bf16 into the chunk's output tile (8 bytes per lane per tile)
  auto finish_output = [&](int co, const bf16x8 (&af)[kTpFrags]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mt = 2 * kb; mt < 4; ++mt) O[mt] = mfma(ub[kb], af[tri_frag(mt, kb)], O[mt]);
    char *ot = &ost[co & 1][32 * wave + 8 * q4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      *reinterpret_cast<u32x2 *>(ot + (16 * mt + r16) * kOPitch) = pack4_bf16(O[mt][0], O[mt][1], O[mt][2], O[mt][3]);
  };
  auto load_scores = [&](int co, bf16x8 (&af)[kTpFrags]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < kTpFrags; ++f) af[f] = __builtin_bit_cast(bf16x8, afb[co & 1][f * 64 + lane]);
  };

  __syncthreads(); // chunk 0 staged

  // One chunk step.  The dependent chain is  split(h) -> K h -> R -> split ->
  // T' R -> uc -> split -> K^T uc -> h.  T' is lower triangular, so rows 0..31
  // of uc (half A) need rows 0..31 of R only: the step runs as two halves, the
  // vector work of one half issuing while the MFMAs of the other run, and the
  // output's products (the previous chunk's A uc, this chunk's Q h) filling
  // the split of h.  Scheduling barriers keep the sections in this order.
  for (int c = 0; c < nch; ++c) {
    GDN_RSTAMP();
    GDN_STAMP(0);
    const Stage &S = st[c & 1];
    const int64_t sl = slot_of(p, s, h, c);
    // entry state: this lane's bf16 h fragments are 8 consecutive dk of column
    // colw + r16, so they leave as 16-byte pieces of the [dv][dk] rows
    uint16_t *edst = kEntry ? p.s_entry + sl * (kDim * kDim) + (colw + r16) * kDim + 8 * q4 : nullptr;

    bf16x8 Hh[4], Hl[4];
    f32x4 Hn[8];
    bf16x8 kB[4][2];
    f32x4 eg[4];
    u32x2 vv[4];
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    // the operands of K h rows 32..63 and of R, issued during the split
    auto load_kb_eg_v = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) kB[kb][mt] = rfrag(S.kr, mt + 2, kb);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        eg[mt] = *reinterpret_cast<const f32x4 *>(S.eg + 16 * mt + 4 * q4);
        // V[16mt + 4q + ii][colw + r16], ii = 0..3: a transposing read of the V rows
        vv[mt] = read_tr(S.vr, vrow_slot(16 * mt + 4 * q4 + (r16 >> 2), 2 * wave + ((r16 & 3) >> 1)) * 16 + 8 * (r16 & 1));
      }
    };
    if constexpr (kOL) {
      // ---- h -> hi/lo (chain order over dk, eight consecutive dk per lane),
      // each pair's bf16 h to ht (the output's h) and, when asked for, out as
      // the entry state; K h rows 0..31 of each pair's dk block issue while
      // the next pair is split
      u32x4 *hto = ht + ((c & 1) * kStrips + wave) * 4 * 64 + lane;
      bf16x8 kA[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) kA[kb][mt] = rfrag(S.kr, mt, kb);
      const float en = S.en[0]; // exp(G_n)
      // exp(G_n) h goes to new registers before each pair is split, so that the
      // split can overwrite h in place
      Hn[0] = H[0] * en;
      Hn[1] = H[1] * en;
      split_tiles(H[0], H[1], m0, m1, Hh[0], Hl[0]);
      hto[0] = __builtin_bit_cast(u32x4, Hh[0]);
      if (kEntry) *reinterpret_cast<u32x4 *>(edst) = __builtin_bit_cast(u32x4, Hh[0]);
      load_kb_eg_v();
      __builtin_amdgcn_sched_barrier(0);
      GDN_STAMP(1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt] = mfma(kA[kb][mt], Hh[kb], acc[mt]);
          acc[mt] = mfma(kA[kb][mt], Hl[kb], acc[mt]);
        }
        if (kb < 3) {
          Hn[2 * kb + 2] = H[2 * kb + 2] * en;
          Hn[2 * kb + 3] = H[2 * kb + 3] * en;
          split_tiles(H[2 * kb + 2], H[2 * kb + 3], m0, m1, Hh[kb + 1], Hl[kb + 1]);
          hto[64 * (kb + 1)] = __builtin_bit_cast(u32x4, Hh[kb + 1]);
          if (kEntry) *reinterpret_cast<u32x4 *>(edst + 32 * (kb + 1)) = __builtin_bit_cast(u32x4, Hh[kb + 1]);
          GDN_INTERLEAVE(4, 6, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      GDN_STAMP(2);
      GDN_STAMP(3);
    } else {
      // ---- h -> hi/lo (chain order over dk, eight consecutive dk per lane);
      // bf16(h) is the entry state.  The previous chunk's output, then Q h, the
      // output's state term, issue among the split's vector instructions.
      bf16x8 kA[4][2], qa[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) kA[kb][mt] = rfrag(S.kr, mt, kb);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) qa[0][mt] = rfrag(S.qr, mt, 0);
      const float en = S.en[0]; // exp(G_n)
      if (c > 0) {
        bf16x8 af[kTpFrags];
        load_scores(c - 1, af);
        finish_output(c - 1, af);
      }
      // exp(G_n) h goes to new registers before each pair is split, so that the
      // split can overwrite h in place
      Hn[0] = H[0] * en;
      Hn[1] = H[1] * en;
      split_tiles(H[0], H[1], m0, m1, Hh[0], Hl[0]);
      if (kEntry) *reinterpret_cast<u32x4 *>(edst) = __builtin_bit_cast(u32x4, Hh[0]);
      __builtin_amdgcn_sched_barrier(0);
      GDN_STAMP(1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) O[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < 3) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) qa[(kb + 1) & 1][mt] = rfrag(S.qr, mt, kb + 1);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) O[mt] = mfma(Hh[kb], qa[kb & 1][mt], O[mt]);
        if (kb < 3) {
          Hn[2 * kb + 2] = H[2 * kb + 2] * en;
          Hn[2 * kb + 3] = H[2 * kb + 3] * en;
          split_tiles(H[2 * kb + 2], H[2 * kb + 3], m0, m1, Hh[kb + 1], Hl[kb + 1]);
          if (kEntry) *reinterpret_cast<u32x4 *>(edst + 32 * (kb + 1)) = __builtin_bit_cast(u32x4, Hh[kb + 1]);
          GDN_INTERLEAVE(4, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      GDN_STAMP(2);

      // ---- K h, half A (rows 0..31), while h is scaled by exp(G_n) ----------
      load_kb_eg_v();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt] = mfma(kA[kb][mt], Hh[kb], acc[mt]);
          acc[mt] = mfma(kA[kb][mt], Hl[kb], acc[mt]);
        }
      GDN_INTERLEAVE(16, 2, 1);
      __builtin_amdgcn_sched_barrier(0);
      GDN_STAMP(3);
    }

    // ---- K h, half B, while R = V - diag(exp(G)) K h of half A is formed ---
    bf16x8 th[kTpFrags], tl[kTpFrags];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      th[tri_frag(mt, 0)] = __builtin_bit_cast(bf16x8, S.tp[tri_frag(mt, 0) * 64 + lane]);
      tl[tri_frag(mt, 0)] = __builtin_bit_cast(bf16x8, S.tp[(kTpFrags + tri_frag(mt, 0)) * 64 + lane]);
    }
    auto form_r = [&](int mt, f32x4 &R) __attribute__((always_inline)) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const uint32_t pr = vv[mt][ii >> 1];
        const float v = __builtin_bit_cast(float, (ii & 1) ? (pr & 0xFFFF0000u) : (pr << 16));
        R[ii] = v - eg[mt][ii] * acc[mt][ii];
      }
    };
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        acc[mt + 2] = mfma(kB[kb][mt], Hh[kb], acc[mt + 2]);
        acc[mt + 2] = mfma(kB[kb][mt], Hl[kb], acc[mt + 2]);
      }
    f32x4 R[4];
    form_r(0, R[0]);
    form_r(1, R[1]);
    bf16x8 Rh[2], Rl[2];
    split_tiles(R[0], R[1], m0, m1, Rh[0], Rl[0]);
    GDN_INTERLEAVE(16, 3, 2);
    __builtin_amdgcn_sched_barrier(0);
    GDN_STAMP(4);

    // ---- uc = T' R: half A (rows 0..31) and the R-A part of half B, while R
    // of half B is formed ----------------------------------------------------
#pragma unroll
    for (int mt = 2; mt < 4; ++mt) {
      th[tri_frag(mt, 1)] = __builtin_bit_cast(bf16x8, S.tp[tri_frag(mt, 1) * 64 + lane]);
      tl[tri_frag(mt, 1)] = __builtin_bit_cast(bf16x8, S.tp[(kTpFrags + tri_frag(mt, 1)) * 64 + lane]);
    }
    // the decays of uc and of the output's state term, two sections ahead of
    // their use
    f32x4 dn[4];
    float dq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      dn[mt] = *reinterpret_cast<const f32x4 *>(S.dn + 16 * mt + 4 * q4);
      if constexpr (!kOL) dq[mt] = S.dq[16 * mt + r16];
    }
    f32x4 D[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      D[mt] = mfma(th[tri_frag(mt, 0)], Rh[0], D[mt]);
      D[mt] = mfma(th[tri_frag(mt, 0)], Rl[0], D[mt]);
      D[mt] = mfma(tl[tri_frag(mt, 0)], Rh[0], D[mt]);
    }
    form_r(2, R[2]);
    form_r(3, R[3]);
    split_tiles(R[2], R[3], m0, m1, Rh[1], Rl[1]);
    GDN_INTERLEAVE(12, 3, 3);
    __builtin_amdgcn_sched_barrier(0);
    GDN_STAMP(5);

    // ---- uc half B (R-B part), while half A of uc is rounded for the output,
    // decayed and split; the output's state term is scaled ------------------
    bf16x8 kt0[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) kt0[m] = ktfrag(S, m, 0);
#pragma unroll
    for (int mt = 2; mt < 4; ++mt) {
      D[mt] = mfma(th[tri_frag(mt, 1)], Rh[1], D[mt]);
      D[mt] = mfma(th[tri_frag(mt, 1)], Rl[1], D[mt]);
      D[mt] = mfma(tl[tri_frag(mt, 1)], Rh[1], D[mt]);
    }
    bf16x8 Dh[2], Dl[2];
    ub[0] = chain_frag(D[0], D[1]);
    if constexpr (kOL) ut[((c & 1) * kStrips + wave) * 2 * 64 + lane] = __builtin_bit_cast(u32x4, ub[0]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) D[mt] *= dn[mt];
    split_tiles(D[0], D[1], m0, m1, Dh[0], Dl[0]);
    if constexpr (!kOL) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) O[mt] *= dq[mt];
    }
    GDN_INTERLEAVE(6, 6, 4);
    __builtin_amdgcn_sched_barrier(0);
    GDN_STAMP(6);

    // ---- h += K^T diag(exp(G_n - G)) uc, half A, while half B of uc is
    // rounded, decayed and split --------------------------------------------
    bf16x8 kt1[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) kt1[m] = ktfrag(S, m, 1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      Hn[m] = mfma(kt0[m], Dh[0], Hn[m]);
      Hn[m] = mfma(kt0[m], Dl[0], Hn[m]);
    }
    ub[1] = chain_frag(D[2], D[3]);
    if constexpr (kOL) ut[((c & 1) * kStrips + wave) * 2 * 64 + 64 + lane] = __builtin_bit_cast(u32x4, ub[1]);
#pragma unroll
    for (int mt = 2; mt < 4; ++mt) D[mt] *= dn[mt];
    split_tiles(D[2], D[3], m0, m1, Dh[1], Dl[1]);
    GDN_INTERLEAVE(16, 2, 5);
    __builtin_amdgcn_sched_barrier(0);
    GDN_STAMP(7);

    // ---- h += ..., half B --------------------------------------------------
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      Hn[m] = mfma(kt1[m], Dh[1], Hn[m]);
      Hn[m] = mfma(kt1[m], Dl[1], Hn[m]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) H[m] = Hn[m];
    GDN_STAMP(8);

    __syncthreads();
    GDN_STAMP(9);
    GDN_STAMP_FLUSH(c);
  }
  // the last chunk's output: its scores were formed in the last step (kOL:
  // a loader forms it in the step this barrier closes)
  if constexpr (!kOL) {
    bf16x8 af[kTpFrags];
    load_scores(nch - 1, af);
    finish_output(nch - 1, af);
  }
  __syncthreads();
#undef GDN_INTERLEAVE

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
  const dim3 block((kStrips + loader_waves<kStrips>()) * 64);
  if (p.opts & kOptEntry)
    hipLaunchKernelGGL((chunk_delta_h_fwd_o<kStrips, true>), dim3(blocks), block, 0, stream, p);
  else
    hipLaunchKernelGGL((chunk_delta_h_fwd_o<kStrips, false>), dim3(blocks), block, 0, stream, p);
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
