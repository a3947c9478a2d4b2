// gdn_api.hip -- the C ABI of include/gdn_prefill.h: argument validation
// (pure host logic), the scratch layout, and the two launches on the caller's
// stream.
//
// Convention from the page "spark_model/layers/ops/ssm_gdn_a3.rs"
// (gdn_tc_spine_reject): every rejection names the guard that rejected, and a
// path that cannot run fails loudly; nothing here falls back to anything.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gdn_prefill.h"
#include "gdn_params.h"

// The scratch of gdn_prefill_noalloc (gc, T' and the row scales of one call):
// a fixed array that every GPU the library runs on holds until the process
// ends.  Host code never passes this name to a kernel -- in host code it is a
// stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, looked up once per device (scratch_on below).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace gdn {
hipError_t launch_stage1(const Params &p, hipStream_t stream);
hipError_t launch_stage2(const Params &p, hipStream_t stream);
hipError_t launch_decode(const Params &p, hipStream_t stream);
} // namespace gdn

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return GDN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void *ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// A dispatch counts its work-items in 32 bits per grid dimension.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

// Grid extents of the two prefill launches (the launchers' own formulas), and
// the int fields of the parameter block, checked before anything is launched.
int check_extents(int B, int T, int nk, int nv, const gdn_varlen *varlen) {
  const int64_t per_seq = varlen ? varlen->max_chunks : (int64_t(T) + GDN_CHUNK - 1) / GDN_CHUNK;
  const int64_t total = varlen ? varlen->total_chunks : int64_t(B) * per_seq;
  if (total > INT32_MAX)
    return fail(GDN_EINVAL, "sizes: B=%d x %lld chunks per sequence exceeds %d chunk slots per head", B,
                (long long)per_seq, INT32_MAX);
  // stage 1: one 64-lane workgroup per (chunk rounded up to 8, v-head)
  if (((per_seq + 7) / 8) * 8 * nv * 64 > kMaxWorkItems)
    return fail(GDN_EINVAL, "sizes: %lld chunks per sequence x nv=%d exceed the stage-1 grid", (long long)per_seq,
                nv);
  // stage 2: at most two 512-lane workgroups per (sequence, v-head) chain, the
  // k-groups rounded up to 8 (one or two strips per workgroup are only chosen
  // when there are fewer chains than compute units)
  if (((int64_t(B) * nk + 7) / 8) * 8 * (nv / nk) * 2 * 512 > kMaxWorkItems)
    return fail(GDN_EINVAL, "sizes: B=%d x nv=%d chains exceed the stage-2 grid", B, nv);
  return GDN_OK;
}

// Chunk slots per head, or -1 when the sizes are invalid.
int64_t chunk_slots(int B, int T, const gdn_varlen *varlen) {
  if (B <= 0) return -1;
  if (varlen) {
    if (varlen->total_chunks < 0 || varlen->max_chunks < 0) return -1;
    return varlen->total_chunks;
  }
  if (T <= 0) return -1;
  return int64_t(B) * ((int64_t(T) + GDN_CHUNK - 1) / GDN_CHUNK);
}

int check_flags(unsigned flags) {
  if (flags & ~unsigned(GDN_OPT_ENTRY_STATES | GDN_OPT_L2NORM_QK))
    return fail(GDN_EINVAL, "flags=0x%x: only GDN_OPT_ENTRY_STATES (0x%x) and GDN_OPT_L2NORM_QK (0x%x) exist", flags,
                unsigned(GDN_OPT_ENTRY_STATES), unsigned(GDN_OPT_L2NORM_QK));
  return GDN_OK;
}

// The regions gc, tp, [nrm], [s_entry] of `slots` chunk slots, from byte 0,
// each 256-byte aligned; absent regions get GDN_NO_REGION.
void place_regions(int64_t slots, unsigned flags, gdn_scratch_layout *out) {
  size_t off = 0;
  out->slots = slots;
  out->flags = flags;
  out->gc = off;
  off = align256(off + size_t(slots) * gdn::kGcBytes);
  out->tp = off;
  off = align256(off + size_t(slots) * gdn::kTpBytes);
  out->nrm = GDN_NO_REGION;
  if (flags & GDN_OPT_L2NORM_QK) {
    out->nrm = off;
    off = align256(off + size_t(slots) * gdn::kNrmBytes);
  }
  out->s_entry = GDN_NO_REGION;
  if (flags & GDN_OPT_ENTRY_STATES) {
    out->s_entry = off;
    off = align256(off + size_t(slots) * gdn::kSBytes);
  }
  out->total = off > 256 ? off : 256; // never 0 for a valid problem
}

int layout(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen, unsigned flags,
           gdn_scratch_layout *out) {
  if (dk != GDN_HEAD_DIM || dv != GDN_HEAD_DIM)
    return fail(GDN_EUNSUPPORTED, "head size: dk=%d dv=%d, the kernels are built for dk = dv = 128", dk, dv);
  if (nv <= 0 || nk <= 0 || nv % nk != 0)
    return fail(GDN_EINVAL, "head counts: nk=%d nv=%d (nv must be a positive multiple of nk)", nk, nv);
  int rc = check_flags(flags);
  if (rc != GDN_OK) return rc;
  const int64_t chunks = chunk_slots(B, T, varlen);
  if (chunks < 0)
    return fail(GDN_EINVAL, "sizes: B=%d T=%d%s give no valid chunk count", B, T,
                varlen ? " (ragged: max_chunks/total_chunks must be >= 0)" : "");
  place_regions(chunks * nv, flags, out);
  return ok();
}

// Every argument check of gdn_prefill_ex except the scratch buffer's.
int validate_args(const void *q, const void *k, const void *v, const float *g, const float *beta, void *h_state,
                  int h_state_is_table, void *out, int B, int T, int nk, int nv, int dk, int dv,
                  const gdn_strides *strides, const gdn_varlen *varlen, unsigned flags) {
  if (dk != GDN_HEAD_DIM || dv != GDN_HEAD_DIM)
    return fail(GDN_EUNSUPPORTED, "head size: dk=%d dv=%d, the kernels are built for dk = dv = 128", dk, dv);
  if (nk <= 0 || nv <= 0) return fail(GDN_EINVAL, "head counts: nk=%d nv=%d must be positive", nk, nv);
  if (nv % nk != 0) return fail(GDN_EINVAL, "GQA grouping: nv=%d is not a multiple of nk=%d", nv, nk);
  if (B <= 0 || B > 65535) return fail(GDN_EINVAL, "B=%d must be in 1..65535", B);
  if (varlen == nullptr && T <= 0) return fail(GDN_EINVAL, "T=%d must be positive for dense input", T);
  if (varlen != nullptr && T < 0) return fail(GDN_EINVAL, "T=%d (total tokens) must be >= 0", T);
  // a ragged call with no tokens reads and writes no token rows
  const bool no_tokens = (varlen != nullptr && T == 0);
  if (!no_tokens && (!q || !k || !v)) return fail(GDN_EINVAL, "null pointer: q, k and v are required");
  if (!no_tokens && (!g || !beta)) return fail(GDN_EINVAL, "null pointer: g and beta are required");
  if (!h_state) return fail(GDN_EINVAL, "null pointer: h_state is required");
  if (!no_tokens && !out) return fail(GDN_EINVAL, "null pointer: out is required");
  if (!strides) return fail(GDN_EINVAL, "null pointer: strides is required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(GDN_EINVAL, "alignment: q, k and v must be 16-byte aligned (16-byte vector loads)");
  if (!aligned(g, 4) || !aligned(beta, 4)) return fail(GDN_EINVAL, "alignment: g and beta must be 4-byte aligned");
  if (!aligned(h_state, h_state_is_table ? 8 : 16))
    return fail(GDN_EINVAL, "alignment: h_state must be 16-byte aligned (8 for a pointer table)");
  if (!aligned(out, 16)) return fail(GDN_EINVAL, "alignment: out must be 16-byte aligned");
  if (h_state_is_table != 0 && h_state_is_table != 1)
    return fail(GDN_EINVAL, "h_state_is_table=%d must be 0 or 1", h_state_is_table);
  if (strides->qk_row % 8 != 0 || strides->v_row % 8 != 0)
    return fail(GDN_EINVAL,
                "strides: qk_row=%lld and v_row=%lld must be multiples of 8 (rows are read 16 bytes at a time)",
                (long long)strides->qk_row, (long long)strides->v_row);
  if (strides->qk_row < int64_t(nk) * GDN_HEAD_DIM)
    return fail(GDN_EINVAL, "strides: qk_row=%lld is smaller than nk*128=%d", (long long)strides->qk_row,
                nk * GDN_HEAD_DIM);
  if (strides->v_row < int64_t(nv) * GDN_HEAD_DIM)
    return fail(GDN_EINVAL, "strides: v_row=%lld is smaller than nv*128=%d", (long long)strides->v_row,
                nv * GDN_HEAD_DIM);
  if (strides->qk_row > GDN_MAX_ROW_PITCH || strides->v_row > GDN_MAX_ROW_PITCH)
    return fail(GDN_EINVAL, "strides: qk_row=%lld and v_row=%lld must not exceed %d elements",
                (long long)strides->qk_row, (long long)strides->v_row, GDN_MAX_ROW_PITCH);
  if (int64_t(nv) * GDN_HEAD_DIM > GDN_MAX_ROW_PITCH)
    return fail(GDN_EINVAL, "head counts: nv=%d makes output rows longer than %d elements", nv, GDN_MAX_ROW_PITCH);
  if (strides->gb_row < nv)
    return fail(GDN_EINVAL, "strides: gb_row=%lld is smaller than nv=%d", (long long)strides->gb_row, nv);
  if (varlen) {
    if (!varlen->cu_seqlens || !varlen->cu_chunks)
      return fail(GDN_EINVAL, "ragged: cu_seqlens and cu_chunks are required");
    if (!aligned(varlen->cu_seqlens, 4) || !aligned(varlen->cu_chunks, 4))
      return fail(GDN_EINVAL, "ragged: cu_seqlens and cu_chunks must be 4-byte aligned");
    if (varlen->max_chunks < 0 || varlen->total_chunks < 0)
      return fail(GDN_EINVAL, "ragged: max_chunks=%d and total_chunks=%d must be >= 0", varlen->max_chunks,
                  varlen->total_chunks);
    if (varlen->max_chunks > varlen->total_chunks)
      return fail(GDN_EINVAL, "ragged: max_chunks=%d exceeds total_chunks=%d", varlen->max_chunks,
                  varlen->total_chunks);
    if (int64_t(varlen->total_chunks) * GDN_CHUNK < int64_t(T))
      return fail(GDN_EINVAL, "ragged: total_chunks=%d cannot hold T=%d tokens", varlen->total_chunks, T);
    // every chunk holds at least one token, so the offsets cannot describe
    // more chunks than tokens (and with T == 0 none at all: the token
    // pointers may then be NULL only because nothing is launched)
    if (int64_t(varlen->total_chunks) > int64_t(T))
      return fail(GDN_EINVAL, "ragged: total_chunks=%d exceeds T=%d tokens (a chunk holds at least one token)",
                  varlen->total_chunks, T);
  }
  int rc = check_flags(flags);
  if (rc != GDN_OK) return rc;
  return check_extents(B, T, nk, nv, varlen);
}

int validate(const void *q, const void *k, const void *v, const float *g, const float *beta,
             void *h_state, int h_state_is_table, void *out, void *scratch, size_t scratch_bytes,
             int B, int T, int nk, int nv, int dk, int dv, const gdn_strides *strides,
             const gdn_varlen *varlen, unsigned flags, gdn_scratch_layout *lay) {
  int rc = validate_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, T, nk, nv, dk, dv, strides, varlen,
                         flags);
  if (rc != GDN_OK) return rc;
  if (!scratch) return fail(GDN_EINVAL, "null pointer: scratch is required");
  if (!aligned(scratch, 256)) return fail(GDN_EINVAL, "alignment: scratch must be 256-byte aligned");
  rc = layout(B, T, nk, nv, dk, dv, varlen, flags, lay);
  if (rc != GDN_OK) return rc;
  if (scratch_bytes < lay->total)
    return fail(GDN_ESCRATCH, "scratch: %zu bytes given, %zu needed", scratch_bytes, lay->total);
  return ok();
}

#ifdef GDN_SECTION_STAMPS
unsigned long long *g_stamps = nullptr; // profiling build: where the spine's section stamps go
#endif

// The parameter block.  scratch holds the regions of `lay`; the entry states
// go to s_entry_out when it is given, else to the scratch's s_entry region.
gdn::Params make_params(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        void *h_state, int h_state_is_table, void *out, void *scratch, int B, int T,
                        int nk, int nv, const gdn_strides *strides, const gdn_varlen *varlen,
                        const gdn_scratch_layout &lay, void *s_entry_out = nullptr) {
  gdn::Params p{};
  unsigned char *base = static_cast<unsigned char *>(scratch);
  p.q = static_cast<const uint16_t *>(q);
  p.k = static_cast<const uint16_t *>(k);
  p.v = static_cast<const uint16_t *>(v);
  p.g = g;
  p.beta = beta;
  p.h_state = h_state;
  p.h_is_table = h_state_is_table;
  p.out = static_cast<uint16_t *>(out);
  p.gc = reinterpret_cast<float *>(base + lay.gc);
  p.tp = reinterpret_cast<uint16_t *>(base + lay.tp);
  p.nrm = lay.nrm == GDN_NO_REGION ? nullptr : reinterpret_cast<float *>(base + lay.nrm);
  if (s_entry_out)
    p.s_entry = static_cast<uint16_t *>(s_entry_out);
  else
    p.s_entry = lay.s_entry == GDN_NO_REGION ? nullptr : reinterpret_cast<uint16_t *>(base + lay.s_entry);
  p.opts = lay.flags;
#ifdef GDN_SECTION_STAMPS
  p.stamps = g_stamps;
#endif
  p.qk_row = strides->qk_row;
  p.v_row = strides->v_row;
  p.gb_row = strides->gb_row;
  p.B = B;
  p.T = T;
  p.nk = nk;
  p.nv = nv;
  if (varlen) {
    p.n_chunks = 0;
    p.max_chunks = varlen->max_chunks;
    p.total_chunks = varlen->total_chunks;
    p.cu_seqlens = varlen->cu_seqlens;
    p.cu_chunks = varlen->cu_chunks;
  } else {
    p.n_chunks = (T + GDN_CHUNK - 1) / GDN_CHUNK;
    p.max_chunks = p.n_chunks;
    p.total_chunks = B * p.n_chunks;
    p.cu_seqlens = nullptr;
    p.cu_chunks = nullptr;
  }
  return p;
}

int run_stage(int stage, const gdn::Params &p, hipStream_t stream) {
  static const char *names[3] = {"", "chunk_cumsum_recompute_wu", "chunk_delta_h_fwd_o"};
  if (p.max_chunks == 0) return ok(); // every sequence is empty: nothing to do
  const hipError_t e = (stage == 1) ? gdn::launch_stage1(p, stream) : gdn::launch_stage2(p, stream);
  if (e != hipSuccess)
    return fail(GDN_EHIP, "launch of %s failed: %s", names[stage], hipGetErrorString(e));
  return ok();
}

// ---- the no-allocation variant ------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev: looked up with dev current, on
// the first call for that device, then kept.
int scratch_on(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_EHIP, "device %d: the no-allocation scratch is kept for devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(GDN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(GDN_EHIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr)
      return fail(GDN_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

int validate_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv,
                    const gdn_strides *strides, unsigned flags) {
  if (flags & ~unsigned(GDN_OPT_L2NORM_QK))
    return fail(GDN_EINVAL, "flags=0x%x: the decode takes only GDN_OPT_L2NORM_QK (0x%x)", flags,
                unsigned(GDN_OPT_L2NORM_QK));
  if (dk != GDN_HEAD_DIM || dv != GDN_HEAD_DIM)
    return fail(GDN_EUNSUPPORTED, "head size: dk=%d dv=%d, the kernels are built for dk = dv = 128", dk, dv);
  if (nk <= 0 || nv <= 0) return fail(GDN_EINVAL, "head counts: nk=%d nv=%d must be positive", nk, nv);
  if (nv % nk != 0) return fail(GDN_EINVAL, "GQA grouping: nv=%d is not a multiple of nk=%d", nv, nk);
  // one 256-lane workgroup (four waves of 32 state rows) per v-head
  if (int64_t(nv) * (GDN_HEAD_DIM / 32) * 64 > kMaxWorkItems)
    return fail(GDN_EINVAL, "nv=%d is too large for the decode grid", nv);
  if (B <= 0 || B > 65535) return fail(GDN_EINVAL, "B=%d must be in 1..65535", B);
  if (!q || !k || !v) return fail(GDN_EINVAL, "null pointer: q, k and v are required");
  if (!g || !beta) return fail(GDN_EINVAL, "null pointer: g and beta are required");
  if (!h_state) return fail(GDN_EINVAL, "null pointer: h_state is required");
  if (!out) return fail(GDN_EINVAL, "null pointer: out is required");
  if (!strides) return fail(GDN_EINVAL, "null pointer: strides is required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(GDN_EINVAL, "alignment: q, k and v must be 16-byte aligned (16-byte vector loads)");
  if (!aligned(g, 4) || !aligned(beta, 4)) return fail(GDN_EINVAL, "alignment: g and beta must be 4-byte aligned");
  if (h_state_is_table != 0 && h_state_is_table != 1)
    return fail(GDN_EINVAL, "h_state_is_table=%d must be 0 or 1", h_state_is_table);
  if (!aligned(h_state, h_state_is_table ? 8 : 16))
    return fail(GDN_EINVAL, "alignment: h_state must be 16-byte aligned (8 for a pointer table)");
  if (!aligned(out, 16)) return fail(GDN_EINVAL, "alignment: out must be 16-byte aligned");
  if (strides->qk_row % 8 != 0 || strides->v_row % 8 != 0)
    return fail(GDN_EINVAL,
                "strides: qk_row=%lld and v_row=%lld must be multiples of 8 (rows are read 16 bytes at a time)",
                (long long)strides->qk_row, (long long)strides->v_row);
  if (strides->qk_row < int64_t(nk) * GDN_HEAD_DIM)
    return fail(GDN_EINVAL, "strides: qk_row=%lld is smaller than nk*128=%d", (long long)strides->qk_row,
                nk * GDN_HEAD_DIM);
  if (strides->v_row < int64_t(nv) * GDN_HEAD_DIM)
    return fail(GDN_EINVAL, "strides: v_row=%lld is smaller than nv*128=%d", (long long)strides->v_row,
                nv * GDN_HEAD_DIM);
  if (strides->gb_row < nv)
    return fail(GDN_EINVAL, "strides: gb_row=%lld is smaller than nv=%d", (long long)strides->gb_row, nv);
  return ok();
}

} // namespace

extern "C" {

size_t gdn_prefill_scratch_bytes_ex(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen,
                                    unsigned flags) {
  gdn_scratch_layout lay;
  if (layout(B, T, nk, nv, dk, dv, varlen, flags, &lay) != GDN_OK) return 0;
  return lay.total;
}

size_t gdn_prefill_scratch_bytes(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen) {
  return gdn_prefill_scratch_bytes_ex(B, T, nk, nv, dk, dv, varlen, GDN_OPT_ENTRY_STATES);
}

int gdn_prefill_scratch_layout_ex(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen,
                                  unsigned flags, gdn_scratch_layout *out) {
  if (!out) return fail(GDN_EINVAL, "null pointer: layout output is required");
  return layout(B, T, nk, nv, dk, dv, varlen, flags, out);
}

int gdn_prefill_scratch_layout(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen,
                               gdn_scratch_layout *out) {
  return gdn_prefill_scratch_layout_ex(B, T, nk, nv, dk, dv, varlen, GDN_OPT_ENTRY_STATES, out);
}

int gdn_prefill_validate_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                            void *h_state, int h_state_is_table, void *out, void *scratch, size_t scratch_bytes,
                            int B, int T, int nk, int nv, int dk, int dv, const gdn_strides *strides,
                            const gdn_varlen *varlen, unsigned flags) {
  gdn_scratch_layout lay;
  return validate(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B, T, nk, nv, dk, dv,
                  strides, varlen, flags, &lay);
}

int gdn_prefill_validate(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         void *h_state, int h_state_is_table, void *out, void *scratch,
                         size_t scratch_bytes, int B, int T, int nk, int nv, int dk, int dv,
                         const gdn_strides *strides, const gdn_varlen *varlen) {
  return gdn_prefill_validate_ex(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B, T,
                                 nk, nv, dk, dv, strides, varlen, GDN_OPT_ENTRY_STATES);
}

int gdn_prefill_stage_ex(int stage, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, void *h_state, int h_state_is_table, void *out, void *scratch,
                         size_t scratch_bytes, int B, int T, int nk, int nv, int dk, int dv,
                         const gdn_strides *strides, const gdn_varlen *varlen, unsigned flags, void *stream) {
  if (stage < 1 || stage > 2) return fail(GDN_EINVAL, "stage=%d must be 1 or 2", stage);
  gdn_scratch_layout lay;
  int rc = validate(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B, T, nk,
                    nv, dk, dv, strides, varlen, flags, &lay);
  if (rc != GDN_OK) return rc;
  const gdn::Params p = make_params(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, B, T, nk,
                                    nv, strides, varlen, lay);
  return run_stage(stage, p, static_cast<hipStream_t>(stream));
}

int gdn_prefill_stage(int stage, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, void *h_state, int h_state_is_table, void *out, void *scratch,
                      size_t scratch_bytes, int B, int T, int nk, int nv, int dk, int dv,
                      const gdn_strides *strides, const gdn_varlen *varlen, void *stream) {
  return gdn_prefill_stage_ex(stage, q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B,
                              T, nk, nv, dk, dv, strides, varlen, GDN_OPT_ENTRY_STATES, stream);
}

int gdn_prefill_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                   void *h_state, int h_state_is_table, void *out, void *scratch, size_t scratch_bytes,
                   int B, int T, int nk, int nv, int dk, int dv, const gdn_strides *strides,
                   const gdn_varlen *varlen, unsigned flags, void *stream) {
  gdn_scratch_layout lay;
  int rc = validate(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B, T, nk,
                    nv, dk, dv, strides, varlen, flags, &lay);
  if (rc != GDN_OK) return rc;
  const gdn::Params p = make_params(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, B, T, nk,
                                    nv, strides, varlen, lay);
  for (int stage = 1; stage <= 2; ++stage) {
    rc = run_stage(stage, p, static_cast<hipStream_t>(stream));
    if (rc != GDN_OK) return rc;
  }
  return GDN_OK;
}

int gdn_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                void *h_state, int h_state_is_table, void *out, void *scratch, size_t scratch_bytes,
                int B, int T, int nk, int nv, int dk, int dv, const gdn_strides *strides,
                const gdn_varlen *varlen, void *stream) {
  return gdn_prefill_ex(q, k, v, g, beta, h_state, h_state_is_table, out, scratch, scratch_bytes, B, T, nk, nv,
                        dk, dv, strides, varlen, GDN_OPT_ENTRY_STATES, stream);
}

int gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        void *h_state, int h_state_is_table, void *out, void *s_entry_out, int B, int T, int nk,
                        int nv, int dk, int dv, const gdn_strides *strides, const gdn_varlen *varlen,
                        unsigned flags, void *stream) {
  int rc = validate_args(q, k, v, g, beta, h_state, h_state_is_table, out, B, T, nk, nv, dk, dv, strides, varlen,
                         flags);
  if (rc != GDN_OK) return rc;
  const bool entry = (flags & GDN_OPT_ENTRY_STATES) != 0;
  if (entry && !s_entry_out)
    return fail(GDN_EINVAL, "null pointer: s_entry_out is required with GDN_OPT_ENTRY_STATES");
  if (entry && !aligned(s_entry_out, 16)) return fail(GDN_EINVAL, "alignment: s_entry_out must be 16-byte aligned");
  // the intermediates only: the entry states are the caller's output
  gdn_scratch_layout lay;
  rc = layout(B, T, nk, nv, dk, dv, varlen, flags & ~unsigned(GDN_OPT_ENTRY_STATES), &lay);
  if (rc != GDN_OK) return rc;
  if (lay.total > GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ESCRATCH,
                "no-allocation scratch: %lld chunk slots need %zu bytes of intermediates, the fixed array holds "
                "%zu; use gdn_prefill_ex with a caller scratch for problems this large",
                (long long)lay.slots, lay.total, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_EHIP, "device of the stream: %s", hipGetErrorString(e));
  void *base = nullptr;
  rc = scratch_on(dev, &base);
  if (rc != GDN_OK) return rc;
  gdn::Params p = make_params(q, k, v, g, beta, h_state, h_state_is_table, out, base, B, T, nk, nv, strides,
                              varlen, lay, entry ? s_entry_out : nullptr);
  p.opts = flags;
  for (int stage = 1; stage <= 2; ++stage) {
    rc = run_stage(stage, p, static_cast<hipStream_t>(stream));
    if (rc != GDN_OK) return rc;
  }
  return GDN_OK;
}

int gdn_varlen_check_host(int B, int T, const int32_t *cu_seqlens_host, const int32_t *cu_chunks_host,
                          int32_t max_chunks, int32_t total_chunks) {
  if (B <= 0) return fail(GDN_EINVAL, "B=%d must be positive", B);
  if (T < 0) return fail(GDN_EINVAL, "T=%d (total tokens) must be >= 0", T);
  if (!cu_seqlens_host || !cu_chunks_host) return fail(GDN_EINVAL, "null pointer: offsets are required");
  if (cu_seqlens_host[0] != 0 || cu_chunks_host[0] != 0)
    return fail(GDN_EINVAL, "ragged: cu_seqlens[0] and cu_chunks[0] must be 0");
  int32_t mx = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t len = int64_t(cu_seqlens_host[i + 1]) - cu_seqlens_host[i];
    const int64_t nch = int64_t(cu_chunks_host[i + 1]) - cu_chunks_host[i];
    if (len < 0) return fail(GDN_EINVAL, "ragged: cu_seqlens decreases at sequence %d", i);
    if (nch != (len + GDN_CHUNK - 1) / GDN_CHUNK)
      return fail(GDN_EINVAL, "ragged: sequence %d has %lld tokens but %lld chunks (needs ceil(len/64))", i,
                  (long long)len, (long long)nch);
    if (nch > mx) mx = int32_t(nch);
  }
  if (cu_seqlens_host[B] != T)
    return fail(GDN_EINVAL, "ragged: cu_seqlens[B]=%d but T=%d tokens", cu_seqlens_host[B], T);
  if (mx != max_chunks)
    return fail(GDN_EINVAL, "ragged: max_chunks=%d but the longest sequence has %d chunks", max_chunks, mx);
  if (cu_chunks_host[B] != total_chunks)
    return fail(GDN_EINVAL, "ragged: total_chunks=%d but cu_chunks[B]=%d", total_chunks, cu_chunks_host[B]);
  return ok();
}

int gdn_decode_validate_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv,
                           const gdn_strides *strides, unsigned flags) {
  return validate_decode(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, flags);
}

int gdn_decode_validate(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv,
                        const gdn_strides *strides) {
  return validate_decode(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, 0u);
}

int gdn_decode_ex(const void *q, const void *k, const void *v, const float *g, const float *beta, void *h_state,
                  int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv, const gdn_strides *strides,
                  unsigned flags, void *stream) {
  int rc = validate_decode(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, flags);
  if (rc != GDN_OK) return rc;
  gdn::Params p{};
  p.q = static_cast<const uint16_t *>(q);
  p.k = static_cast<const uint16_t *>(k);
  p.v = static_cast<const uint16_t *>(v);
  p.g = g;
  p.beta = beta;
  p.h_state = h_state;
  p.h_is_table = h_state_is_table;
  p.out = static_cast<uint16_t *>(out);
  p.qk_row = strides->qk_row;
  p.v_row = strides->v_row;
  p.gb_row = strides->gb_row;
  p.B = B;
  p.T = 1;
  p.nk = nk;
  p.nv = nv;
  p.opts = flags;
  const hipError_t e = gdn::launch_decode(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDN_EHIP, "launch of recurrent_decode failed: %s", hipGetErrorString(e));
  return ok();
}

int gdn_decode(const void *q, const void *k, const void *v, const float *g, const float *beta, void *h_state,
               int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv, const gdn_strides *strides,
               void *stream) {
  return gdn_decode_ex(q, k, v, g, beta, h_state, h_state_is_table, out, B, nk, nv, dk, dv, strides, 0u, stream);
}

const char *gdn_last_error(void) { return g_err; }

#ifdef GDN_SECTION_STAMPS
// Profiling build only: the device buffer (kStampWaves * kStampSteps *
// kStampSlots 64-bit words) that the spine's workgroup 0 stamps; NULL stops it.
// The stamps are written only while a buffer is set.
void gdn_debug_set_stamps(void *buf) { g_stamps = static_cast<unsigned long long *>(buf); }
#endif

} // extern "C"
