// Decode: one recurrent step of the gated delta rule per sequence -- the step
// that follows a prefill, on the state the prefill leaves in place (page
// "spark_model/layers/ops/ssm_gdn_a3.rs", gdn_prefill_fla's doc comment: the
// final state is updated in place, one state per request).  For
// each (sequence, v-head), with h the stored state ([dk][dv] = S^T), a =
// exp(g) and k, q of the v-head's k-head:
//   delta = beta (v - a h^T k)                (dv)
//   h    <- a h + k delta^T
//   o     = h^T q = a (h_old^T q) + (k . q) delta
// A workgroup of four waves owns one head: wave w holds rows 32w .. 32w+31
// of h, all 128 columns, 64 floats per lane, so that every load and store
// moves two whole 512-byte rows.  The sums over dk (h^T k, h^T q, k . q) are
// formed per wave in registers and with a lane shuffle, then combined across
// the four waves through LDS (4 KB, one barrier); each wave then updates its
// rows and writes them back once: 128 KB of HBM traffic per head, the bound
// of this kernel.  (One wave per 32-column block, the four blocks of a head
// in separate workgroups, moved 128-byte row pieces instead and ran 10 %
// slower.)
// With q/k normalisation (kNorm) the same exchange also sums |k|^2 and |q|^2
// over the waves' rows; with sk = 1/|k|, sq = 1/|q| (0 for a zero vector) the
// sums become sk h^T k, sq h^T q and sk sq k . q, and h takes sk k delta^T:
// the step on k/|k| and q/|q|, the prefill's normalisation.
#include "gdn_device.h"

namespace gdn {

constexpr int kDecWaves = 4; // waves per workgroup (one head): 32 rows each

template <bool kNorm>
__global__ __launch_bounds__(64 * kDecWaves) void recurrent_decode(Params p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x, i = blockIdx.y;
  const int kh = (h * p.nk) / p.nv;
  // wave w holds rows 32w .. 32w+31 of the head's state, all 128 columns: load
  // j (0..15) is rows 32w + 2j and 32w + 2j + 1, whole 512-byte rows, lane l
  // columns 4 (l % 32) .. +3 of row 32w + 2j + l / 32
  const int rsub = lane >> 5, col = 4 * (lane & 31);
  const int row0 = 32 * w + rsub;

  float *hp = state_of(p, i, h);
  f32x4 H[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) H[j] = *reinterpret_cast<const f32x4 *>(hp + (row0 + 2 * j) * kDim + col);

  // k and q of this lane's rows (32w + 2j + rsub): the wave's 64-byte slices
  // of the k and q rows, read whole by every lane
  const uint16_t *qrow = p.q + int64_t(i) * p.qk_row + int64_t(kh) * kDim + 32 * w;
  const uint16_t *krow = p.k + int64_t(i) * p.qk_row + int64_t(kh) * kDim + 32 * w;
  float kr[16], qr[16];
#pragma unroll
  for (int j4 = 0; j4 < 4; ++j4) {
    const u32x4 kv = *reinterpret_cast<const u32x4 *>(krow + 8 * j4);
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(qrow + 8 * j4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { // elements 8 j4 + 2e and + 1: rows 2j and 2j + 1, j = 4 j4 + e
      const uint32_t kw = kv[e], qw = qv[e];
      kr[4 * j4 + e] = bf16_bits_to_f32(rsub ? (kw >> 16) : (kw & 0xFFFFu));
      qr[4 * j4 + e] = bf16_bits_to_f32(rsub ? (qw >> 16) : (qw & 0xFFFFu));
    }
  }
  const float g = p.g[int64_t(i) * p.gb_row + h];
  const float beta = p.beta[int64_t(i) * p.gb_row + h];
  const float a = expf(g);

  // h^T k, h^T q and k . q over the wave's 32 rows, then over the waves
  f32x4 hk = zero4(), hq = zero4();
  float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    hk += H[j] * kr[j];
    hq += H[j] * qr[j];
    kq += kr[j] * qr[j];
    if (kNorm) {
      kk += kr[j] * kr[j];
      qq += qr[j] * qr[j];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hk[e] += __shfl_xor(hk[e], 32, 64);
    hq[e] += __shfl_xor(hq[e], 32, 64);
  }
  // over the two row halves; the 32 column lanes hold the same sums
  kq += __shfl_xor(kq, 32, 64);
  if (kNorm) {
    kk += __shfl_xor(kk, 32, 64);
    qq += __shfl_xor(qq, 32, 64);
  }
  __shared__ f32x4 part[kDecWaves][2][32];
  __shared__ float kqp[kDecWaves][3];
  if (lane < 32) {
    part[w][0][lane] = hk;
    part[w][1][lane] = hq;
  }
  if (lane == 0) {
    kqp[w][0] = kq;
    if (kNorm) {
      kqp[w][1] = kk;
      kqp[w][2] = qq;
    }
  }
  __syncthreads();
  hk = zero4();
  hq = zero4();
  kq = 0.f;
  kk = 0.f;
  qq = 0.f;
#pragma unroll
  for (int u = 0; u < kDecWaves; ++u) {
    hk += part[u][0][lane & 31];
    hq += part[u][1][lane & 31];
    kq += kqp[u][0];
    if (kNorm) {
      kk += kqp[u][1];
      qq += kqp[u][2];
    }
  }
  float sk = 1.f;
  if (kNorm) {
    sk = kk > 0.f ? rsqrtf(kk) : 0.f;
    const float sq = qq > 0.f ? rsqrtf(qq) : 0.f;
    hk *= sk;
    hq *= sq;
    kq *= sk * sq;
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
    *reinterpret_cast<f32x4 *>(hp + (row0 + 2 * j) * kDim + col) = a * H[j] + (sk * kr[j]) * delta;

  if (w == 0 && rsub == 0)
    *reinterpret_cast<u32x2 *>(p.out + (int64_t(i) * p.nv + h) * kDim + col) = pack4_bf16(o[0], o[1], o[2], o[3]);
}

hipError_t launch_decode(const Params &p, hipStream_t stream) {
  dim3 grid(unsigned(p.nv), p.B);
  if (p.opts & kOptNorm)
    hipLaunchKernelGGL(recurrent_decode<true>, grid, dim3(64 * kDecWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(recurrent_decode<false>, grid, dim3(64 * kDecWaves), 0, stream, p);
  return hipGetLastError();
}

} // namespace gdn
