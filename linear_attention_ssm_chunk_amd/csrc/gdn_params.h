// gdn_params.h -- one parameter block shared by the host launcher and the two
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
constexpr int64_t kDecBytes = int64_t(2) * kChunk * 4;   // exp(G_t), exp(G_{n-1} - G_t)
// T' per slot: float16, the six fragments in order f, 8 values (16 bytes) per
// lane; the two diagonal fragments (f = 0, 4) keep only their first 4 (8
// bytes): their other half is the zero block above the diagonal.
constexpr int64_t kTpBytes = (4 * 16 + 2 * 8) * 64;        // 5 KB
constexpr bool tp_half(int f) { return f == 0 || f == 4; }
constexpr int tp_offset(int f) {          // byte offset of fragment f
  return f == 0 ? 0 : f == 1 ? 512 : f == 2 ? 1536 : f == 3 ? 2560 : f == 4 ? 3584 : 4096;
}
constexpr int64_t kSBytes = int64_t(kDim) * kDim * 2;    // entry state, bf16 [dv][dk]

struct Params {
  // inputs (bf16 as raw 16-bit patterns)
  const uint16_t *q, *k, *v;
  const float *g, *beta;
  // state: contiguous [B][nv][dk][dv] or a device table of B pointers
  void *h_state;
  int h_is_table;
  uint16_t *out; // bf16 [N_tok][nv][dv]
  // scratch regions
  float *gc, *dec;
  uint16_t *tp, *s_entry;
  int64_t qk_row, v_row, gb_row; // token-row pitches in elements
  int B, T, nk, nv;
  int n_chunks;                  // dense: ceil(T/64)
  int max_chunks, total_chunks;  // grid extent, chunk slots per head
  const int32_t *cu_seqlens, *cu_chunks; // NULL = dense
};

} // namespace gdn
