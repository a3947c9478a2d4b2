// gdn_device.h -- device helpers for the gfx950 kernels: MFMA fragments,
// bf16 conversion and the sequence / slot bookkeeping shared by all stages.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_bf16, wave64; lane l,
// r = l % 16, q = l / 16):
//   A (16 x 32): lane holds row r, eight k values
//   B (32 x 16): lane holds column r, eight k values
//   C (16 x 16): lane holds column r, rows 4q .. 4q+3
// The k order inside a lane is free as long as A and B use the same one.  Two
// orders are used:
//   contiguous  element e <-> k = 8q + e             (operands read from memory)
//   chain       element e <-> k = 4q + e      (e < 4)
//                             k = 16 + 4q + e - 4 (e >= 4)
// The chain order makes the C fragments of two vertically stacked 16x16
// tiles an operand of the next product without moving data between lanes:
// registers (tile 2j, tile 2j+1) of a C result are exactly the k = 32j..32j+31
// block of a B (or, read as its transpose, an A) operand.
// Where a tile is needed in the other orientation, the kernels read it from
// LDS with the transposing read ds_read_b64_tr_b16 (K^T and V in the spine, the
// entry states on their way out), or form the product transposed (the
// spine's output, O^T = h^T Q^T + uc^T A^T).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_params.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
// Two floats -> one register of two bf16 (a in the low half), one instruction.
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Pack four floats (consecutive elements of one lane) as 4 bf16 = 8 bytes.
__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  return u32x2{cvt_pk(a, b), cvt_pk(c, d)};
}

// Chain-order fragment from two C tiles (tile for k 0..15 and k 16..31).
__device__ __forceinline__ bf16x8 chain_frag(const f32x4 &lo_tile, const f32x4 &hi_tile) {
  return __builtin_bit_cast(bf16x8, u32x4{cvt_pk(lo_tile[0], lo_tile[1]), cvt_pk(lo_tile[2], lo_tile[3]),
                                          cvt_pk(hi_tile[0], hi_tile[1]), cvt_pk(hi_tile[2], hi_tile[3])});
}

// The dk order of the spine.  Row rho = 16m + 4q + i of the state tiles
// (m = 0..7, q, i = 0..3) holds dk = perm_dk(rho) = 32(m/2) + 8q + 4(m%2) + i.
// Then the chain fragment of tiles (2kb, 2kb+1) gives a lane eight consecutive
// dk, 32kb + 8q .. +7: K and Q rows are read, and entry states written, as
// 16-byte pieces, and the contiguous k order of a row fragment is this order.
__host__ __device__ constexpr int perm_dk(int rho) {
  return 32 * (rho >> 5) + 8 * ((rho >> 2) & 3) + 4 * ((rho >> 4) & 1) + (rho & 3);
}

// Fragment slot of a lower-triangular 64x64 A operand (T', the scores) held as
// 16x32 fragments (mt, kb): only mt >= 2kb can be nonzero, six in all.
__host__ __device__ constexpr int tri_frag(int mt, int kb) { return kb == 0 ? mt : mt + 2; }

__device__ __forceinline__ bf16x8 load16_bf16x8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Where a sequence lives.  Ragged offsets are checked here so that a bad table
// skips the sequence instead of reading or writing outside the caller's token
// rows (cu_seqlens within [0, T]) or the scratch (cu_chunks within
// [0, total_chunks]).
struct Seq {
  int64_t tok0;   // first token row
  int len;        // tokens
  int64_t chunk0; // first chunk slot (per head)
  int nchunks;
  bool ok;
};

__device__ __forceinline__ Seq seq_of(const Params &p, int i) {
  Seq s;
  if (p.cu_seqlens == nullptr) {
    s.tok0 = int64_t(i) * p.T;
    s.len = p.T;
    s.chunk0 = int64_t(i) * p.n_chunks;
    s.nchunks = p.n_chunks;
    s.ok = true;
  } else {
    const int a = p.cu_seqlens[i], b = p.cu_seqlens[i + 1];
    const int ca = p.cu_chunks[i], cb = p.cu_chunks[i + 1];
    s.tok0 = a;
    s.len = b - a;
    s.chunk0 = ca;
    s.nchunks = cb - ca;
    s.ok = (a >= 0) && (s.len >= 0) && (b <= p.T) && (ca >= 0) && (cb <= p.total_chunks) &&
           (s.nchunks == (s.len + kChunk - 1) / kChunk) && (s.nchunks <= p.max_chunks);
  }
  return s;
}

// Chunk slot of (sequence s, v-head h, chunk c): [seq][head][chunk] order.
__device__ __forceinline__ int64_t slot_of(const Params &p, const Seq &s, int h, int c) {
  return s.chunk0 * p.nv + int64_t(h) * s.nchunks + c;
}

__device__ __forceinline__ float *state_of(const Params &p, int i, int h) {
  if (p.h_is_table) {
    float *base = reinterpret_cast<float *const *>(p.h_state)[i];
    return base + int64_t(h) * kDim * kDim;
  }
  return reinterpret_cast<float *>(p.h_state) + (int64_t(i) * p.nv + h) * kDim * kDim;
}

} // namespace gdn
