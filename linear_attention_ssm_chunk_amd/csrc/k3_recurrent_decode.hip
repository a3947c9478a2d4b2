// Decode: one recurrent step of the gated delta rule per sequence -- the step
// that follows a prefill, on the state the prefill leaves in place (page
// "spark_model/layers/ops/ssm_gdn_a3.rs", gdn_prefill_fla's doc comment: the
// final state is updated in place, one state per request).  For
// each (sequence, v-head), with h the stored state ([dk][dv] = S^T), a =
// exp(g) and k, q of the v-head's k-head:
//   delta = beta (v - a h^T k)                (dv)
//   h    <- a h + k delta^T
//   o     = h^T q = a (h_old^T q) + (k . q) delta
// The dv columns are independent, so a workgroup (one wave) owns one 32-column
// block of one head: 128 rows x 32 columns of float32, 64 per lane.  The block
// is read once (8 rows of 128 contiguous bytes per load), reduced over dk in
// registers and with lane shuffles, updated, and written back once: 32 KB of
// HBM traffic per block, the bound of this kernel.
#include "gdn_device.h"

namespace gdn {

constexpr int kDecCols = 32; // columns per workgroup

__global__ __launch_bounds__(64) void recurrent_decode(Params p) {
  const int cb = blockIdx.x & 3;           // column block
  const int h = blockIdx.x >> 2, i = blockIdx.y;
  const int kh = (h * p.nk) / p.nv;
  const int lane = threadIdx.x;
  const int c4 = lane & 7;  // this lane's 4 columns: cb*32 + 4*c4 .. +3
  const int rg = lane >> 3; // this lane's rows: rg + 8j, j = 0..15
  const int col = cb * kDecCols + 4 * c4;

  float *hp = state_of(p, i, h);
  f32x4 H[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) H[j] = *reinterpret_cast<const f32x4 *>(hp + (rg + 8 * j) * kDim + col);

  // k and q: every lane reads the whole 256-byte rows (the same addresses for
  // all lanes) and keeps element rg of each 8-element piece: rows rg + 8j
  const uint16_t *qrow = p.q + int64_t(i) * p.qk_row + int64_t(kh) * kDim;
  const uint16_t *krow = p.k + int64_t(i) * p.qk_row + int64_t(kh) * kDim;
  float kr[16], qr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const u32x4 kv = *reinterpret_cast<const u32x4 *>(krow + 8 * j);
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(qrow + 8 * j);
    const uint32_t kw = kv[rg >> 1], qw = qv[rg >> 1];
    kr[j] = bf16_bits_to_f32((rg & 1) ? (kw >> 16) : (kw & 0xFFFFu));
    qr[j] = bf16_bits_to_f32((rg & 1) ? (qw >> 16) : (qw & 0xFFFFu));
  }
  const float g = p.g[int64_t(i) * p.gb_row + h];
  const float beta = p.beta[int64_t(i) * p.gb_row + h];
  const float a = expf(g);

  // h^T k and h^T q over this lane's rows, then over the 8 row groups
  f32x4 hk = zero4(), hq = zero4();
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    hk += H[j] * kr[j];
    hq += H[j] * qr[j];
    kq += kr[j] * qr[j];
  }
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hk[e] += __shfl_xor(hk[e], m, 64);
      hq[e] += __shfl_xor(hq[e], m, 64);
    }
    kq += __shfl_xor(kq, m, 64);
  }

  // delta for the lane's columns; v of this head
  const u32x2 vw = *reinterpret_cast<const u32x2 *>(p.v + int64_t(i) * p.v_row + int64_t(h) * kDim + col);
  const float v4[4] = {bf16_bits_to_f32(vw[0] & 0xFFFFu), bf16_bits_to_f32(vw[0] >> 16),
                       bf16_bits_to_f32(vw[1] & 0xFFFFu), bf16_bits_to_f32(vw[1] >> 16)};
  f32x4 delta, o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    delta[e] = beta * (v4[e] - a * hk[e]);
    o[e] = a * hq[e] + kq * delta[e];
  }

  // h <- a h + k delta^T, written back in place
#pragma unroll
  for (int j = 0; j < 16; ++j)
    *reinterpret_cast<f32x4 *>(hp + (rg + 8 * j) * kDim + col) = a * H[j] + kr[j] * delta;

  if (rg == 0)
    *reinterpret_cast<u32x2 *>(p.out + (int64_t(i) * p.nv + h) * kDim + col) = pack4_bf16(o[0], o[1], o[2], o[3]);
}

hipError_t launch_decode(const Params &p, hipStream_t stream) {
  dim3 grid(unsigned(p.nv) * (kDim / kDecCols), p.B);
  hipLaunchKernelGGL(recurrent_decode, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
