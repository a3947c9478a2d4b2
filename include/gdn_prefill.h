/*
 * gdn_prefill.h -- C ABI of the MI355X (gfx950) chunked gated-delta-rule
 * (Gated DeltaNet) prefill forward.
 *
 * The operation.  Per value head, over the tokens of each sequence,
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t                                    (no query scale)
 * -- the gated delta rule, which the page "spark_model/layers/ops/ssm_gdn_a3.rs"
 * runs as its GDN prefill (its kernels are the gated_delta_rule_chunk_* family).
 * It is evaluated in 64-token chunks in the three stages that page lists in the
 * doc comment of gdn_prefill_fla, run as two kernels:
 *   1. chunk_cumsum_recompute_wu: chunk-local cumulative log-gate gc, the
 *      strictly lower L (sharing the key Gram), and the WY/UT solves
 *      (I+L) W = beta exp(gc) K, (I+L) U = beta V -- emitted as the UT
 *      transform T' = (I+L)^-1 diag(beta), which gives U = T' V and
 *      W = T' diag(exp(gc)) K;
 *   2. chunk_delta_h_fwd_o: the serial float32 state spine over chunks (the
 *      page's chunk_delta_h), which emits each chunk's entry state, forms the
 *      corrected values uc = U - W h (= T' (V - diag(exp(gc)) K h)), and leaves
 *      the final state in place -- with the page's stage 3, chunk_fwd_o,
 *      O = diag(exp(gc)) Q h_c + tril(decay * Q K^T) uc, formed in the same
 *      pass while h_c and uc are still in registers.
 * The arguments follow that page's launcher (gdn_prefill_fla's parameter
 * list): separate k/v head counts, packed strided rows, optional ragged
 * cu_seqlens / cu_chunks, a per-request state pointer table, caller-owned
 * scratch, one stream.
 *
 * Conventions.
 *   - dk = dv = 128 and the chunk is 64 tokens (the kernels are specialised,
 *     as the page's tile guard gdn_tc_spine_reject is); other sizes are
 *     rejected with GDN_EUNSUPPORTED.
 *   - GQA grouping: v-head h reads k-head (h * nk) / nv; nv % nk == 0.
 *   - The state is stored h[dk][dv] (as the page's h_state: nv states per
 *     request, key dimension first), the transpose of S above.
 *   - Tokens of a sequence occupy consecutive token rows.  Dense mode:
 *     sequence b is rows b*T .. b*T+T-1.  Ragged mode: rows cu_seqlens[i] ..
 *     cu_seqlens[i+1]-1.
 *   - Element (row, head h, component d) of q / k is at
 *     q[row*qk_row + kappa(h)*128 + d]; of v at v[row*v_row + h*128 + d];
 *     g and beta at g[row*gb_row + h], beta[row*gb_row + h].  Strides are in
 *     ELEMENTS.  q, k and v may point into one packed buffer (the page's conv
 *     layout: qk_stride = v_stride = conv_dim, gb_stride = 2*nv).
 *   - out is bf16 [N_tok][nv][dv], contiguous (N_tok = B*T, or cu_seqlens[B]).
 *   - exp(gc) of the chunk-local gate must stay finite in float32 (gc < 88);
 *     g <= 0 (a decay) always satisfies it, and any decay however strong is
 *     handled (factors that underflow are 0, as they are in the result).
 *   - The method normalises q and k per token to unit length.  By default the
 *     caller passes them normalised; with GDN_OPT_L2NORM_QK the kernels do it
 *     (k / |k|, q / |q| per token and k-head; a zero vector stays zero).
 *     T' = (I+L)^-1 diag(beta) is bounded in the method's domain: with
 *     beta_t |k_t|^2 <= rho < 2, 0 <= beta_t <= beta_max and g <= 0,
 *     |T'_rs| <= ||T'||_2 <= 2 beta_max / (2 - rho), so <= 2 for unit keys and
 *     beta in [0, 1].  It passes between the kernels as an exact bf16 hi + lo
 *     pair (float32's exponent range, ~2^-17 relative), so no T' of finite
 *     inputs overflows on the way.
 *
 * Ownership.  The caller owns every buffer.  The library allocates nothing,
 * keeps no pointer after return, and never reads device memory from the host.
 * q, k, v, g, beta may alias each other (read-only).  out, scratch and the
 * state must not alias the inputs or each other.
 *
 * Execution.  gdn_prefill enqueues two kernels on `stream` (a hipStream_t)
 * and returns; there is no device synchronisation.  Asynchronous faults
 * surface at the caller's next synchronisation.  Calls on different streams
 * with disjoint outputs and scratch may run concurrently.
 *
 * Errors.  Every entry point returns GDN_OK (0) or a negative code;
 * gdn_last_error() then names the guard that rejected the call (thread-local
 * text).  There is no fallback path of any kind.
 */
#ifndef GDN_PREFILL_H
#define GDN_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_CHUNK 64
#define GDN_HEAD_DIM 128
/* Largest token-row pitch (qk_row, v_row, and nv*128 of out), in elements: the
 * kernels address the 64 rows of a chunk with 32-bit byte offsets. */
#define GDN_MAX_ROW_PITCH (1 << 24)

enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,       /* malformed argument (null pointer, bad stride, ...) */
  GDN_EUNSUPPORTED = -2, /* head size / chunk other than 128 / 64            */
  GDN_ESCRATCH = -3,     /* scratch_bytes smaller than gdn_prefill_scratch_bytes */
  GDN_EHIP = -4          /* a HIP runtime call failed; message has its text  */
};

/* Options of the *_ex calls (bit flags).  The calls without _ex use
 * GDN_OPT_ENTRY_STATES. */
#define GDN_OPT_ENTRY_STATES 0x1u /* emit every chunk's entry state (scratch region s_entry) */
#define GDN_OPT_L2NORM_QK 0x2u    /* normalise q and k to unit length inside the kernels     */

/* Token-row pitches in elements (the page's qk_stride, v_stride, gb_stride). */
typedef struct gdn_strides {
  int64_t qk_row; /* q and k rows (bf16 elements); multiple of 8, <= GDN_MAX_ROW_PITCH */
  int64_t v_row;  /* v rows (bf16 elements); multiple of 8, <= GDN_MAX_ROW_PITCH       */
  int64_t gb_row; /* g and beta rows (float elements); >= nv     */
} gdn_strides;

/* Ragged co-dispatch (the page's VARLEN arguments).  Pass NULL for dense. */
typedef struct gdn_varlen {
  const int32_t *cu_seqlens; /* device, B+1 token offsets, cu_seqlens[0] = 0     */
  const int32_t *cu_chunks;  /* device, B+1 chunk offsets,
                                cu_chunks[i+1]-cu_chunks[i] = ceil(len_i / 64)   */
  int32_t max_chunks;        /* host: max_i ceil(len_i / 64) (grid extent)       */
  int32_t total_chunks;      /* host: cu_chunks[B] (sizes the scratch)           */
} gdn_varlen;

/*
 * Scratch layout (the page's caller-owned, pre-sized scratch that the launcher
 * sub-divides: gdn_prefill_fla's doc comment, BufferArena gdn_fla_scratch).  A
 * "slot" is one (sequence, v-head, chunk):
 *   slot(i, h, c) = cu_chunks[i]*nv + h*n_i + c,   n_i = chunks of sequence i
 * (dense: cu_chunks[i] = i*ceil(T/64), so slots run [B][nv][n_chunks]).
 * Regions (byte offsets from the scratch base, each 256-byte aligned; a region
 * the options leave out has offset GDN_NO_REGION and takes no bytes):
 *   gc      float [slots][64]        chunk-local cumulative log-gate G_t; rows
 *                                    past the sequence end repeat the last value
 *   tp      bf16  [slots][2][2560]   the UT transform T' = (I+L)^-1 diag(beta)
 *                                    (so U = T' V, W = T' diag(exp(G)) K) as
 *                                    hi = bf16(T'), then lo = bf16(T' - hi), each
 *                                    in MFMA fragment order.  Of the 16x32
 *                                    fragments (mt, kb) (rows 16mt..,
 *                                    columns 32kb..) only the lower-triangular
 *                                    six, mt >= 2kb, are stored, in the order
 *                                    f = mt for kb = 0 and f = mt + 2 for
 *                                    kb = 1; lane l = 16q + r of fragment f
 *                                    holds row t = 16mt + r, columns
 *                                    s = 32kb + 4q + e (e = 0..3) and
 *                                    s = 32kb + 16 + 4q + e, as 8 values per
 *                                    lane (512 elements per fragment), except
 *                                    the diagonal fragments f = 0 and f = 4
 *                                    (mt = 2kb), which hold only the first 4
 *                                    per lane (256 elements): their other
 *                                    columns lie above the diagonal.  Element
 *                                    offsets of f = 0..5 within a part: 0, 256,
 *                                    768, 1280, 1792, 2048
 *   nrm     float [slots][2][64]     GDN_OPT_L2NORM_QK only: 1/|k_t|, then
 *                                    1/|q_t| (0 for a zero vector)
 *   s_entry bf16  [slots][128][128]  GDN_OPT_ENTRY_STATES only: the state on
 *                                    entry to each chunk (the page's S_out,
 *                                    stage 2) as S = h^T, [dv][dk] -- the
 *                                    recurrence's orientation, transposed from
 *                                    h_state's [dk][dv]: the kernel holds a lane's
 *                                    state as 8 consecutive dk of one dv column,
 *                                    which leave as whole 16-byte pieces of the
 *                                    [dv][dk] rows (the [dk][dv] store measured
 *                                    10% slower on the spine); dense input:
 *                                    [B][nv][T/64][dv][dk]
 */
#define GDN_NO_REGION ((size_t)-1)
typedef struct gdn_scratch_layout {
  size_t gc, tp, nrm, s_entry; /* byte offsets (GDN_NO_REGION: absent) */
  size_t total;                /* bytes needed                          */
  int64_t slots;               /* chunk slots                           */
  unsigned flags;              /* the options the layout is for         */
} gdn_scratch_layout;

/* Scratch bytes for a problem (at least 256), for the given options: the
 * size of the caller's pre-sized scratch (page "spark_model/layers/ops/
 * ssm_gdn_a3.rs", gdn_prefill_fla's doc comment).  varlen NULL: dense B x T.
 * Returns 0 if the sizes or flags are invalid. */
size_t gdn_prefill_scratch_bytes_ex(int B, int T, int nk, int nv, int dk, int dv,
                                    const gdn_varlen *varlen, unsigned flags);
size_t gdn_prefill_scratch_bytes(int B, int T, int nk, int nv, int dk, int dv,
                                 const gdn_varlen *varlen);

/* Fill *out with the scratch layout above (same page and passage).  Returns
 * GDN_OK or an error. */
int gdn_prefill_scratch_layout_ex(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen,
                                  unsigned flags, gdn_scratch_layout *out);
int gdn_prefill_scratch_layout(int B, int T, int nk, int nv, int dk, int dv, const gdn_varlen *varlen,
                               gdn_scratch_layout *out);

/*
 * Validate every argument of gdn_prefill(_ex) without touching the GPU (pure
 * host logic; pointer values are checked for NULL and alignment only).
 * Returns GDN_OK or the code gdn_prefill would return, with the rejecting
 * guard named in gdn_last_error() -- the page's rule for its spine guard
 * (gdn_tc_spine_reject: pure, testable without a GPU, names the guard that
 * rejected).
 */
int gdn_prefill_validate_ex(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, void *h_state, int h_state_is_table, void *out,
                            void *scratch, size_t scratch_bytes, int B, int T, int nk, int nv,
                            int dk, int dv, const gdn_strides *strides, const gdn_varlen *varlen,
                            unsigned flags);
int gdn_prefill_validate(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, void *h_state, int h_state_is_table, void *out,
                         void *scratch, size_t scratch_bytes, int B, int T, int nk, int nv,
                         int dk, int dv, const gdn_strides *strides, const gdn_varlen *varlen);

/*
 * The prefill forward: the page's gdn_prefill_fla (its doc comment and
 * parameter list), stages 1-3 as two launches on one stream.
 *   q, k, v     bf16 device pointers (see Conventions for addressing).
 *   g, beta     float device pointers.
 *   h_state     float state, read as the initial state and OVERWRITTEN with
 *               the final state.  h_state_is_table == 0: contiguous
 *               [B][nv][dk][dv].  == 1: a device array of B device pointers,
 *               entry i -> [nv][dk][dv] of sequence i (the page's pointer
 *               table, one state per request).  The entries live in device
 *               memory, so no call can check them: each must point to
 *               nv*dk*dv writable floats (16-byte aligned) that no other entry
 *               overlaps; the entry of a length-0 sequence is never read.
 *   out         bf16 [N_tok][nv][dv].
 *   scratch     device buffer (256-byte aligned) of >=
 *               gdn_prefill_scratch_bytes(_ex)(...) bytes; on return it holds
 *               the intermediates in the documented layout (the entry states
 *               in region s_entry).
 *   B, T        dense: B sequences of T tokens.  Ragged: B sequences, T is the
 *               total token count cu_seqlens[B]: sequences must lie within
 *               rows [0, T) (the kernels skip any sequence whose offsets leave
 *               [0, T) or the scratch); the host checks total_chunks <= T and
 *               total_chunks * 64 >= T.  With T == 0 (so no chunks) the token
 *               pointers (q, k, v, g, beta, out) may be NULL.
 *   flags       (_ex) GDN_OPT_* options; gdn_prefill uses GDN_OPT_ENTRY_STATES.
 *   stream      hipStream_t.
 * A ragged sequence of length 0 leaves its state unchanged and writes nothing.
 * Size limits (GDN_EINVAL beyond them): 1 <= B <= 65535; chunk slots per head
 * (B * ceil(T/64), or total_chunks) <= INT32_MAX; ceil8(chunks of the longest
 * sequence) * nv * 64 < 2^32 and ceil8(B * nk) * (nv/nk) * 1024 < 2^32 (the
 * two launches count work-items in 32 bits).
 */
int gdn_prefill_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                   void *h_state, int h_state_is_table, void *out, void *scratch,
                   size_t scratch_bytes, int B, int T, int nk, int nv, int dk, int dv,
                   const gdn_strides *strides, const gdn_varlen *varlen, unsigned flags, void *stream);
int gdn_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                void *h_state, int h_state_is_table, void *out, void *scratch,
                size_t scratch_bytes, int B, int T, int nk, int nv, int dk, int dv,
                const gdn_strides *strides, const gdn_varlen *varlen, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gdn_prefill_ex
 * without a caller scratch buffer.  The call's intermediates (regions gc, tp
 * and, with GDN_OPT_L2NORM_QK, nrm of the scratch layout) go to a fixed array of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends; problems whose intermediates need more are rejected with
 * GDN_ESCRATCH (128 MiB holds about 12 700 chunk slots: 64-token chunks times
 * v-heads).  With GDN_OPT_ENTRY_STATES the entry states go to s_entry_out, the
 * caller's output of slots x 128 x 128 bf16 (16-byte aligned; [slot][dv][dk]
 * as region s_entry, slots numbered as in the scratch layout); without it
 * s_entry_out is not read.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * Every call on one GPU uses that GPU's one array and leaves its last contents
 * there, so calls that overlap on a GPU (different streams or host threads)
 * race: the caller serialises them.  The first call on a device looks the
 * array's device address up, with that device current.  Arguments, checks and
 * errors are otherwise those of gdn_prefill_ex.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        void *h_state, int h_state_is_table, void *out, void *s_entry_out, int B, int T,
                        int nk, int nv, int dk, int dv, const gdn_strides *strides,
                        const gdn_varlen *varlen, unsigned flags, void *stream);

/*
 * One kernel of gdn_prefill(_ex) (stage 1 or 2), same arguments, same
 * validation: the page runs its stages as sequential launches on one stream
 * (gdn_prefill_fla's doc comment), and so can a caller.  Stage 2 reads what
 * stage 1 left in scratch; running 1 then 2 on one stream is exactly
 * gdn_prefill(_ex).  For callers that time or interleave the kernels.
 */
int gdn_prefill_stage_ex(int stage, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, void *h_state, int h_state_is_table, void *out,
                         void *scratch, size_t scratch_bytes, int B, int T, int nk, int nv, int dk,
                         int dv, const gdn_strides *strides, const gdn_varlen *varlen, unsigned flags,
                         void *stream);
int gdn_prefill_stage(int stage, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, void *h_state, int h_state_is_table, void *out,
                      void *scratch, size_t scratch_bytes, int B, int T, int nk, int nv, int dk,
                      int dv, const gdn_strides *strides, const gdn_varlen *varlen,
                      void *stream);

/*
 * Host-side check of ragged offsets already copied to host memory (the page's
 * VARLEN arguments of gdn_prefill_fla: cu_seqlens token offsets, cu_chunks
 * chunk offsets, the grid's chunk count the maximum over sequences):
 * cu_seqlens non-decreasing from 0 to cu_seqlens[B] = T,
 * cu_chunks[i+1]-cu_chunks[i] = ceil(len_i/64), max_chunks and total_chunks
 * consistent.  gdn_prefill cannot read device offsets without synchronising,
 * so it trusts them; callers that build offsets at run time can check them
 * here first.  The kernels still skip any sequence whose offsets leave rows
 * [0, T) or chunk slots [0, total_chunks).
 */
int gdn_varlen_check_host(int B, int T, const int32_t *cu_seqlens_host, const int32_t *cu_chunks_host,
                          int32_t max_chunks, int32_t total_chunks);

/*
 * One recurrent step per sequence (decode): the token that follows a prefill,
 * on the state the prefill leaves in place.  For each sequence b and v-head h
 * (k-head kappa = (h * nk) / nv), with S the state, a = exp(g):
 *     S <- a S (I - beta k k^T) + beta v k^T,     o = S q
 * -- the recurrence of the header comment for one token (the gated delta
 * rule; page "spark_model/layers/ops/ssm_gdn_a3.rs", gdn_prefill_fla's doc
 * comment for the in-place state and its per-request table).  In the stored
 * orientation h = S^T: delta = beta (v - a h^T k), h <- a h + k delta^T,
 * o = h^T q.
 *   q, k     bf16; token b's head kappa at q + b*qk_row + kappa*128.
 *   v        bf16; head h at v + b*v_row + h*128.
 *   g, beta  float at g[b*gb_row + h], beta[b*gb_row + h].
 *   h_state  as for gdn_prefill (contiguous [B][nv][dk][dv], or a device
 *            table of B pointers to [nv][dk][dv], each entry 16-byte aligned
 *            as there; every entry is read), updated in place.
 *   out      bf16 [B][nv][dv], contiguous.
 *   flags    (_ex) GDN_OPT_L2NORM_QK: q and k arrive unnormalised and the
 *            kernel takes the step on k/|k| and q/|q| (per token and k-head;
 *            a zero vector stays zero), as gdn_prefill_ex does with that
 *            option, so a sequence prefilled with it decodes the same way.
 *            No other bit is accepted (GDN_EINVAL).  gdn_decode passes 0.
 * dk = dv = 128; 1 <= B <= 65535; nv * 256 < 2^32 (work-items of the launch).  No scratch; one launch on `stream`, no synchronisation.
 * Returns GDN_OK or an error as gdn_prefill does; gdn_decode_validate(_ex)
 * runs the same checks without touching the GPU.
 */
int gdn_decode_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv,
                  const gdn_strides *strides, unsigned flags, void *stream);
int gdn_decode(const void *q, const void *k, const void *v, const float *g, const float *beta,
               void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk, int dv,
               const gdn_strides *strides, void *stream);

int gdn_decode_validate_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk,
                           int dv, const gdn_strides *strides, unsigned flags);
int gdn_decode_validate(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        void *h_state, int h_state_is_table, void *out, int B, int nk, int nv, int dk,
                        int dv, const gdn_strides *strides);

/* Text of the last error on the calling thread ("" after success): the guard
 * that rejected the call, named as the page asks of every rejection
 * (gdn_tc_spine_reject's doc comment). */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PREFILL_H */
