// stream_mix.hip -- the achievable HBM rate for a given read:write mix, for the
// measurements only (compiled into the section-stamp profiling build,
// libgdn_prefill_stamps.so; the product library does not contain it).
//
// One launch reads read_bytes from src and writes write_bytes to dst at the
// same time: workgroup w of the grid streams its share of both ranges with
// 16-byte loads and stores (64-lane coalesced), the loads folded into one word
// per lane so that they cannot be dropped, and that word stored only if it
// equals a value the data never produces.  The spine's own mix (reads q, k,
// v, T', gc, the state; writes o, the entry states, the state) is what the
// caller passes in.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_mix(const u32x4s *__restrict__ src, int64_t n_read,
                                                  u32x4s *__restrict__ dst, int64_t n_write,
                                                  unsigned *__restrict__ sink) {
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
  // kr reads and kw writes per thread, interleaved in proportion (a read
  // whenever the reads are behind their share), so that both streams are in
  // flight together in the ratio of their sizes
  const int64_t kr = (n_read + nthreads - 1) / nthreads, kw = (n_write + nthreads - 1) / nthreads;
  unsigned acc = 0u;
  const u32x4s val = {unsigned(tid), 0x9E3779B9u, unsigned(tid >> 32), 0x7F4A7C15u};
  int64_t r = 0, w = 0;
  for (int64_t s = 0; s < kr + kw; ++s) {
    if (r < kr && (w >= kw || r * kw <= w * kr)) {
      const int64_t i = r * nthreads + tid;
      if (i < n_read) {
        const u32x4s x = src[i];
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
      }
      ++r;
    } else {
      const int64_t i = w * nthreads + tid;
      if (i < n_write) dst[i] = val;
      ++w;
    }
  }
  if (acc == 0xDEADBEEFu) sink[0] = acc; // never taken for the caller's data; keeps the loads
}

} // namespace

extern "C" int gdn_debug_stream_mix(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                                    void *sink, int blocks, void *stream) {
  if (!src || !dst || !sink || read_bytes < 0 || write_bytes < 0 || blocks <= 0 || (read_bytes % 16) ||
      (write_bytes % 16))
    return -1;
  hipLaunchKernelGGL(stream_mix, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4s *>(src), read_bytes / 16, static_cast<u32x4s *>(dst), write_bytes / 16,
                     static_cast<unsigned *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
