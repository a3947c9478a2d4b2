// gdn_params.h -- one parameter block shared by the host launcher and the
// kernels, so the two sides cannot disagree about sizes or layouts (the page
// "spark_model/layers/ops/ssm_gdn_a3.rs" makes the same point about its
// shared-memory footprint constant GDN_TC_SMEM).
#pragma once

#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;    // tokens per chunk
constexpr int kDim = 128;     // dk = dv

// Bytes per chunk slot of each scratch region (see include/gdn_prefill.h).
constexpr int kTpFrags = 6;                              // nonzero 16x32 fragments of T' (lower triangle)
constexpr int64_t kGcBytes = int64_t(kChunk) * 4;        // G_t
constexpr int64_t kNrmBytes = int64_t(2) * kChunk * 4;   // 1/|k_t|, 1/|q_t| (with q/k normalisation)
// T' per slot: bf16 hi, then bf16 lo, each the six fragments in order f, 8
// values (16 bytes) per lane; the two diagonal fragments (f = 0, 4) keep only
// their first 4 (8 bytes): their other half is the zero block above the
// diagonal.
constexpr int64_t kTpHalfBytes = (4 * 16 + 2 * 8) * 64;   // 5 KB per part
constexpr int64_t kTpBytes = 2 * kTpHalfBytes;            // hi + lo
constexpr bool tp_half(int f) { return f == 0 || f == 4; }
constexpr int tp_offset(int f) {          // byte offset of fragment f in a part
  return f == 0 ? 0 : f == 1 ? 512 : f == 2 ? 1536 : f == 3 ? 2560 : f == 4 ? 3584 : 4096;
}
constexpr int64_t kSBytes = int64_t(kDim) * kDim * 2;    // entry state, bf16 [dk][dv]

// Option bits (the GDN_OPT_* values of include/gdn_prefill.h).
constexpr unsigned kOptEntry = 1u;   // emit per-chunk entry states
constexpr unsigned kOptNorm = 2u;    // L2-normalise q and k per token and k-head

struct Params {
  // inputs (bf16 as raw 16-bit patterns)
  const uint16_t *q, *k, *v;
  const float *g, *beta;
  // state: contiguous [B][nv][dk][dv] or a device table of B pointers
  void *h_state;
  int h_is_table;
  uint16_t *out; // bf16 [N_tok][nv][dv]
  // scratch regions (nrm and s_entry only with their options)
  float *gc, *nrm;
  uint16_t *tp, *s_entry;
  int64_t qk_row, v_row, gb_row; // token-row pitches in elements
  int B, T, nk, nv;
  int n_chunks;                  // dense: ceil(T/64)
  int max_chunks, total_chunks;  // grid extent, chunk slots per head
  const int32_t *cu_seqlens, *cu_chunks; // NULL = dense
  unsigned opts;                 // kOptEntry | kOptNorm
#ifdef GDN_SECTION_STAMPS
  // section-stamp profiling build only: clock stamps of workgroup 0's waves
  unsigned long long *stamps;
#endif
};

#ifdef GDN_SECTION_STAMPS
// Steps kStampFirst .. kStampFirst + kStampSteps - 1 of workgroup 0 are
// stamped; each wave has kStampSteps rows of kStampSlots stamps.
constexpr int kStampFirst = 8, kStampSteps = 32, kStampSlots = 16, kStampWaves = 8;
#endif

} // namespace gdn
