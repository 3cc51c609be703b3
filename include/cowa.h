/*
 * cowa.h - C ABI of libcowa, a gfx950 (MI355X) implementation of CoWindow
 * Attention (CoWA): prefill, decode and the prefill's backward.
 *
 * The method.  "CoWindow Attention: Full Causal Coverage Is a Collective
 * Property" (Abstract) and "Splitting long-range windows across KV heads
 * beats duplicating them at lower cost" (mechanism paragraph) describe causal
 * GQA attention in which every KV head sees a shared prefix-sink window and a
 * shared near-diagonal window, while the rest of the causal history is split
 * into non-overlapping long-range intervals, one per KV head, so that the
 * union over heads covers the whole causal prefix.  A head's softmax
 * normalises over the keys that head sees and no others (same news page,
 * paragraph on what CoWA does not claim).  The pattern is computed from
 * positions and the global KV-head index alone (news page, efficiency and
 * tensor-parallelism paragraphs).
 *
 * The pages give no formula; this library fixes the band partition as:
 *     L = ceil((n_ctx - W) / h_kv_global)   if n_ctx > W, else L = 0
 *     vis_g(t, j) = j <= t && ( j < S || t - j < W ||
 *                               (L > 0 && W + g*L <= t - j < W + (g+1)*L) )
 * for query position t, key position j and global KV-head index g.  Query
 * head hq uses local KV head h = hq / (H_q / H_kv_local) and
 * g = kv_head_offset + h.  In COWA_MODE_CAUSAL, vis(t, j) = j <= t (the dense
 * FullAttn comparison, Abstract).
 *
 * Pattern variants on the same kernels:
 *  - n_bands = m < h_kv_global: the duplicated-window ablation of the news
 *    page (ablation paragraph: 1, 2, 4, 8 distinct long-range windows over 8
 *    KV heads at fixed per-head width).  Head g takes window b = g mod m,
 *    i.e. distances [W + b*L, W + (b+1)*L) with the same L as above.
 *  - COWA_MODE_SINK_LOCAL: no long-range window (L = 0), i.e. sliding-window
 *    attention with sinks, the related band-less pattern ("Sliding Window
 *    Attention Beats Linear Attention ...", SWA with attention sinks).
 *
 * Conventions.
 *  - Every device pointer is owned by the caller.  The library never
 *    allocates or frees device memory and never synchronises; work is
 *    enqueued on the given stream (a hipStream_t passed as void*, NULL for
 *    the null stream).
 *  - Host-side validation returns an error before anything is launched.  A
 *    failed launch returns COWA_ERR_HIP.  Nothing throws across the ABI.
 *  - Empty inputs: every count (B, N, H_q, H_kv_local, n_max, n_seqs,
 *    total_tokens, max_seqlen) must be at least 1, else COWA_ERR_INVALID_ARG
 *    and nothing runs.  Inside a packed (varlen) batch a sequence may be
 *    empty (cu_seqlens[b+1] == cu_seqlens[b]); it produces no rows.
 *  - bf16 means IEEE bfloat16 stored as 2 bytes.  Strides are in elements;
 *    the last (head-dim) axis is always contiguous.
 *  - Alignment: the kernels move 16 bytes per lane at the start of every
 *    row, so every tensor base pointer (q, k, v, o, dO, dq, dk, dv, caches,
 *    windowed caches, new tokens) must be 16-byte aligned and every batch,
 *    token and head stride a multiple of 16 bytes (8 bf16 or 4 fp32
 *    elements); otherwise COWA_ERR_INVALID_ARG before any launch.  The
 *    forward also needs 64 token strides of K below 2^30 elements and
 *    d * (N rounded up to 64) below 2^30 (COWA_ERR_UNSUPPORTED otherwise).
 *  - The library is thread-safe.  Its only state is per-thread caches of
 *    plan sizes and launch-order choices per shape, which change no result.
 */
#ifndef COWA_H
#define COWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COWA_OK = 0,
  COWA_ERR_INVALID_ARG = 1,   /* a size, pointer or pattern field is invalid */
  COWA_ERR_UNSUPPORTED = 2,   /* valid but not compiled (head dim, tile shape, group size) */
  COWA_ERR_WORKSPACE = 3,     /* workspace missing, misaligned or too small */
  COWA_ERR_PLAN_MISMATCH = 4, /* plan size does not match pattern/shape/tile */
  COWA_ERR_HIP = 5,           /* a HIP launch failed */
  COWA_ERR_CAPACITY = 6,      /* caller's plan buffers are too small */
  COWA_ERR_SCRATCH_LIMIT = 7  /* needs more than the library's built-in scratch */
} cowa_status;

enum { COWA_MODE_COWA = 0, COWA_MODE_CAUSAL = 1, COWA_MODE_SINK_LOCAL = 2 };
enum { COWA_DTYPE_BF16 = 0, COWA_DTYPE_F32 = 1 };

/* Position-only pattern (mechanism paragraph of the news page; Abstract).
 *  n_ctx          context length the band width is derived from (for decode
 *                 the configured maximum context, so the pattern is the
 *                 same in training and inference)
 *  sink           S >= 0: keys j < S are visible to every head
 *  window         W >= 1: distances t - j < W are visible to every head
 *  band           L; <= 0 means derive L from n_ctx, window, h_kv_global
 *  h_kv_global    KV heads over all tensor-parallel ranks (>= 1)
 *  kv_head_offset global index of this caller's first KV head (tensor
 *                 parallelism keeps the bands complementary across ranks)
 *  mode           COWA_MODE_COWA, COWA_MODE_CAUSAL or COWA_MODE_SINK_LOCAL
 *  n_bands        distinct long-range windows, 0 <= n_bands <= h_kv_global;
 *                 0 means h_kv_global (CoWA proper) */
typedef struct {
  int32_t n_ctx;
  int32_t sink;
  int32_t window;
  int32_t band;
  int32_t h_kv_global;
  int32_t kv_head_offset;
  int32_t mode;
  int32_t n_bands;
} cowa_pattern;

/* Human-readable name of a status code (static storage).  A library utility:
 * the pages define no error model. */
const char* cowa_status_str(cowa_status s);

/* Resolved band width L of a pattern, or -1 if the pattern is invalid.  L is
 * the length of each KV head's long-range interval: the pages split the
 * history beyond the local window into one non-overlapping interval per KV
 * head ("Splitting long-range windows across KV heads beats duplicating them
 * at lower cost", mechanism paragraph) without a formula; this library's
 * formula is the one at the top of this header: the pattern's own band if it
 * sets one, else ceil((n_ctx - W) / h_kv_global) (0 when n_ctx <= W), and 0
 * in COWA_MODE_SINK_LOCAL. */
int32_t cowa_band_length(const cowa_pattern* p);

/* Tile shape (block_m query rows x block_n keys) that cowa_fwd requires for
 * head dim d; COWA_ERR_UNSUPPORTED if d is not compiled (64 and 128 are).  A
 * property of these kernels, not of the method: the visible-tile lists the
 * pages describe as position arithmetic (news page, efficiency paragraph) are
 * built for this tile shape. */
cowa_status cowa_fwd_block_sizes(int32_t d, int32_t* block_m, int32_t* block_n);

/* ---- cowa_visible_ranges: the keys one query row sees (host only) -------
 * The visible keys of query position t for local KV head h (global index
 * g = kv_head_offset + h), as three disjoint half-open key ranges in
 * ascending order: [lo[0], hi[0]) the sink, [lo[1], hi[1]) the long-range
 * window (the keys of the head's band that the sink and the local window do
 * not already hold) and [lo[2], hi[2]) the local window; an empty range has
 * lo == hi.  In COWA_MODE_CAUSAL range 2 is [0, t+1) and the others are
 * empty.  The pattern is position arithmetic only (news page, mechanism
 * paragraph; Abstract: shared windows plus one band per KV head).  The decode
 * kernels evaluate the same function on the device for t = len - 1, so a
 * caller can see exactly which cache rows a decode step reads (and which it
 * will never read again).
 * COWA_ERR_INVALID_ARG for an invalid pattern, h outside
 * [0, h_kv_global - kv_head_offset), t < 0 or a null lo / hi. */
cowa_status cowa_visible_ranges(const cowa_pattern* p, int32_t h, int32_t t, int32_t lo[3],
                                int32_t hi[3]);

/* ---- cowa_plan: visible-tile lists (host only, no device work) ----------
 * For local KV heads h = 0..h_kv_local-1 (global g = kv_head_offset + h) and
 * query tiles qi = 0..ceil(n/block_m)-1, lists the key tiles kj whose block
 * [kj*block_n, (kj+1)*block_n) x rows [qi*block_m, (qi+1)*block_m) holds at
 * least one visible (t, j) with t, j < n.  No router or content is involved:
 * the lists are position arithmetic (news page, efficiency paragraph).
 * Output is CSR in caller host memory:
 *   row_ptr  int32[h_kv_local * nqt + 1], row r = h * nqt + qi
 *   col      int32[nnz], ascending key-tile index within each row
 *   flags    uint8[nnz], 1 if every (t, j) of the tile is visible (the
 *            kernel then skips masking), 0 otherwise; a tile reaching past n
 *            is never full.
 * cowa_plan_size writes nnz; cowa_plan fails with COWA_ERR_CAPACITY if
 * cap < nnz.  n is the number of query rows and of keys (self-attention). */
cowa_status cowa_plan_size(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                           int32_t block_m, int32_t block_n, int64_t* nnz_out);
cowa_status cowa_plan(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                      int32_t block_m, int32_t block_n,
                      int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t cap);

/* ---- cowa_fwd: prefill forward ------------------------------------------
 * O[b,t,hq,:] = sum_{j in vis_g(t)} softmax_j(scale * q.k_j) v_j  and
 * LSE[b,hq,t] = log sum_{j in vis_g(t)} exp(scale * q.k_j)  (natural log),
 * i.e. a softmax over the head's own visible set (news page, paragraph on
 * what CoWA does not claim).
 *  plan        d_row_ptr/d_col/d_flags: device copies of cowa_plan's output
 *              for (p, N, H_kv_local, block_m, block_n); nnz its length.
 *              COWA_ERR_PLAN_MISMATCH if nnz differs from cowa_plan_size.
 *              That length is the only check (the plan is on the device and
 *              the library never reads it back): a plan built for other
 *              arguments with the same length, or altered after cowa_plan,
 *              gives undefined results.
 *  q           bf16 [B, N, H_q, d] with element strides strides[0..2] (b,t,h)
 *  k, v        bf16 [B, N, H_kv_local, d], strides[3..5] and strides[6..8]
 *  o           [B, N, H_q, d] of o_dtype (COWA_DTYPE_BF16 or _F32),
 *              strides[9..11]
 *  lse         fp32 [B, H_q, N], contiguous
 *  d           64 or 128; H_q % H_kv_local == 0;
 *              kv_head_offset + H_kv_local <= h_kv_global
 *  softmax_scale  > 0 (usually 1/sqrt(d))
 *  workspace   caller-owned device memory, 256-byte aligned, at least
 *              cowa_fwd_workspace_size(B, N, H_kv_local, d) bytes, else
 *              COWA_ERR_WORKSPACE.  The call writes V into it head-dim-major
 *              (one row of keys per head dimension) before the attention
 *              kernel reads it; its contents need no initialisation and are
 *              overwritten by every call.  Calls that overlap in time need
 *              separate workspaces.
 * Arithmetic: bf16 inputs, fp32 accumulation and softmax; P is rounded to
 * bf16 before the P.V product. */
cowa_status cowa_fwd(const cowa_pattern* p,
                     const int32_t* d_row_ptr, const int32_t* d_col, const uint8_t* d_flags,
                     int64_t nnz, int32_t block_m, int32_t block_n,
                     const void* q, const void* k, const void* v,
                     void* o, int32_t o_dtype, float* lse,
                     int32_t B, int32_t N, int32_t H_q, int32_t H_kv_local, int32_t d,
                     const int64_t strides[12], float softmax_scale,
                     void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of cowa_fwd for B sequences of N keys (cowa_fwd_varlen:
 * B = n_seqs, N = max_seqlen) with H_kv_local KV heads of dimension d:
 * B * H_kv_local * d * (N rounded up to 64) bf16 values, rounded up to 256
 * bytes.  COWA_ERR_INVALID_ARG for a non-positive size or a null bytes,
 * COWA_ERR_UNSUPPORTED for d other than 64 and 128. */
cowa_status cowa_fwd_workspace_size(int32_t B, int32_t N, int32_t H_kv_local, int32_t d,
                                    size_t* bytes);

/* Packed ("varlen") prefill: n_seqs sequences of different lengths back to
 * back in one launch, a second workload shape of the same operator (used in
 * training and inference, "CoWindow Attention: Full Causal Coverage Is a
 * Collective Property", Abstract).  Sequence b is at token rows
 * [cu_seqlens[b], cu_seqlens[b+1]) of q, o [total_tokens, H_q, d] and k, v
 * [total_tokens, H_kv_local, d]; positions t restart at 0 in every sequence.
 *  cu_seqlens     device int32[n_seqs + 1], cu_seqlens[0] = 0, nondecreasing,
 *                 last = total_tokens, every length <= max_seqlen (not
 *                 checked on the host: rows past max_seqlen are not computed)
 *  plan           cowa_plan for n = max_seqlen (one plan serves every length:
 *                 visibility depends on positions only)
 *  lse            fp32 [H_q, total_tokens]
 *  strides        element strides (t, h) of q, k, v, o (8)
 *  workspace      as for cowa_fwd, at least
 *                 cowa_fwd_workspace_size(n_seqs, max_seqlen, H_kv_local, d). */
cowa_status cowa_fwd_varlen(const cowa_pattern* p, const int32_t* d_row_ptr,
                            const int32_t* d_col, const uint8_t* d_flags, int64_t nnz,
                            int32_t block_m, int32_t block_n, const void* q, const void* k,
                            const void* v, void* o, int32_t o_dtype, float* lse,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                            int32_t total_tokens, int32_t H_q, int32_t H_kv_local, int32_t d,
                            const int64_t strides[8], float softmax_scale,
                            void* workspace, size_t ws_bytes, void* stream);

/* ---- cowa_decode: one query token per sequence --------------------------
 * Sequence b's new token sits at position t_b = cache_seqlens[b] - 1 (its own
 * K/V are already in the cache) and attends to vis_g(t_b) among cached keys
 * 0..t_b; only those keys are read.  The same pattern as prefill is used, as
 * the pages require the pattern to be identical in training and inference
 * (Abstract).  The work is split over chunks of the visible keys of each
 * (b, KV head); a second kernel merges the chunks by log-sum-exp.
 *  q              bf16 [B, H_q, d], strides[0..1] (b, h)
 *  k_cache,v_cache bf16 [B, n_max, H_kv_local, d], strides[2..4], [5..7] (b,s,h)
 *  cache_seqlens  device int32[B], each in [1, n_max] (not checked on the
 *                 host; the kernels clamp to that range)
 *  o              [B, H_q, d] of o_dtype, strides[8..9] (b, h)
 *  lse            fp32 [B, H_q], contiguous
 *  workspace      device scratch of at least cowa_decode_workspace_size bytes
 *                 (256-byte aligned), else COWA_ERR_WORKSPACE; no
 *                 initialisation needed.  Calls that share a workspace must
 *                 not overlap (enqueue them on one stream).
 *  H_q / H_kv_local must be <= 8 (COWA_ERR_UNSUPPORTED otherwise). */
cowa_status cowa_decode_workspace_size(const cowa_pattern* p, int32_t B, int32_t H_q,
                                       int32_t H_kv_local, int32_t d, int32_t n_max,
                                       size_t* bytes);
cowa_status cowa_decode(const cowa_pattern* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_seqlens,
                        void* o, int32_t o_dtype, float* lse,
                        int32_t B, int32_t H_q, int32_t H_kv_local, int32_t d, int32_t n_max,
                        const int64_t strides[10], float softmax_scale,
                        void* workspace, size_t ws_bytes, void* stream);

/* ---- cowa_decode_noalloc: cowa_decode without a workspace ---------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as cowa_decode, minus the workspace: the
 * split partials live in a scratch array the library owns,
 * COWA_DECODE_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends.  The call allocates and frees nothing; its
 * first call on a device (with that device current) looks up the device's
 * copy of the array.
 *  COWA_ERR_SCRATCH_LIMIT when cowa_decode_workspace_size for the same
 *  arguments exceeds COWA_DECODE_SCRATCH_BYTES (the 128K decode workload,
 *  B = 16, H_q = 40, d = 128, needs 10.2 MB), checked before anything runs.
 *  Every call on one GPU uses that GPU's single array: calls that overlap in
 *  time on one GPU (different streams, or threads without ordering) race
 *  and give wrong results; enqueue them on one stream. */
#define COWA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
cowa_status cowa_decode_noalloc(const cowa_pattern* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* cache_seqlens,
                                void* o, int32_t o_dtype, float* lse,
                                int32_t B, int32_t H_q, int32_t H_kv_local, int32_t d,
                                int32_t n_max, const int64_t strides[10],
                                float softmax_scale, void* stream);

/* ---- windowed KV cache for decode ---------------------------------------
 * Per-rank decode memory well below FullAttn's ("CoWindow Attention: Full
 * Causal Coverage Is a Collective Property", Abstract) follows from the
 * pattern: local KV head h (long-range window b = g mod n_bands, g its global
 * index) never again reads a non-sink key at distance >= W + (b+1) L from the
 * newest query.  Its retained cache is S' = min(S, n_max) sink rows followed by
 * a ring of R_h = min(W + (b+1) L, n_max - S') rows; position j >= S' lives in
 * ring row (j - S') mod R_h.  A sequence's windowed cache stacks the local
 * heads in order: rows_h = S' + R_h rows each, every row d contiguous bf16
 * values; k_win and v_win are [B, total_rows, d] with a per-sequence stride
 * (elements) of at least total_rows * d.  COWA_MODE_CAUSAL keeps everything
 * and returns COWA_ERR_UNSUPPORTED. */

/* Rows per local head (head_rows[h_kv_local], may be NULL) and per sequence. */
cowa_status cowa_kv_window_rows(const cowa_pattern* p, int32_t h_kv_local, int32_t n_max,
                                int32_t* head_rows, int64_t* total_rows);

/* Pack the retained rows of full caches [B, n_max, H_kv_local, d] (strides[0..5]:
 * k b,t,h and v b,t,h) for lengths cache_seqlens (device int32[B]) into k_win,
 * v_win (strides[6], strides[7]: their per-sequence strides).  Ring rows that
 * hold no position yet are zeroed. */
cowa_status cowa_kv_window_fill(const cowa_pattern* p, const void* k_cache,
                                const void* v_cache, const int32_t* cache_seqlens,
                                void* k_win, void* v_win, int32_t B, int32_t H_kv_local,
                                int32_t d, int32_t n_max, const int64_t strides[8],
                                void* stream);

/* Write one new token per sequence: k_new, v_new [B, H_kv_local, d] (strides[0..3]:
 * k b,h and v b,h) go to position cache_seqlens[b] - 1 (the length after the
 * append); strides[4], strides[5]: per-sequence strides of k_win, v_win. */
cowa_status cowa_kv_window_append(const cowa_pattern* p, const void* k_new, const void* v_new,
                                  const int32_t* cache_seqlens, void* k_win, void* v_win,
                                  int32_t B, int32_t H_kv_local, int32_t d, int32_t n_max,
                                  const int64_t strides[6], void* stream);

/* cowa_decode against windowed caches: same result as cowa_decode on the full
 * caches the windowed ones were built from.  strides: q b,h; k_win b; v_win b;
 * o b,h.  Workspace as cowa_decode_workspace_size. */
cowa_status cowa_decode_window(const cowa_pattern* p, const void* q, const void* k_win,
                               const void* v_win, const int32_t* cache_seqlens, void* o,
                               int32_t o_dtype, float* lse, int32_t B, int32_t H_q,
                               int32_t H_kv_local, int32_t d, int32_t n_max,
                               const int64_t strides[6], float softmax_scale, void* workspace,
                               size_t ws_bytes, void* stream);

/* ---- cowa_bwd: backward of the prefill (training) operator -------------
 * The pages report the backward latency of the training operator next to
 * the forward ("CoWindow Attention: Full Causal Coverage Is a Collective
 * Property", Abstract).  Gradients of sum(O * dO) with
 *   P_tj = exp(scale q_t.k_j - LSE_t) on vis_g(t), 0 elsewhere,
 *   D_t = sum_c dO_tc O_tc,  dS_tj = P_tj (dO_t.v_j - D_t),
 *   dQ_t = scale sum_j dS_tj k_j,
 *   dK_j = scale sum_{t, hq in group} dS_tj q_t,  dV_j = sum_{t, hq} P_tj dO_t.
 * Two plans of the same pattern are needed:
 *   query-major: cowa_plan with cowa_fwd_block_sizes (the forward plan), for dQ;
 *   key-major:   cowa_plan_kv with cowa_bwd_block_sizes, for dK and dV.
 *  q, k, v, dout  bf16, layouts as in cowa_fwd (dout like q)
 *  o              forward output [B, N, H_q, d] of o_dtype (bf16 or fp32)
 *  lse            forward LSE fp32 [B, H_q, N]
 *  dq             [B, N, H_q, d]; dk, dv [B, N, H_kv_local, d]; all of g_dtype
 *  strides        element strides (b, t, h) of q, k, v, o, dout, dq, dk, dv (24)
 *  workspace      device scratch of cowa_bwd_workspace_size bytes (256-byte
 *                 aligned; no initialisation needed)
 *  d              64 or 128 (COWA_ERR_UNSUPPORTED otherwise).
 * Arithmetic: bf16 operands, fp32 accumulation; P and dS are rounded to bf16
 * before their products. */
cowa_status cowa_bwd_block_sizes(int32_t d, int32_t* block_m, int32_t* block_n);

/* Key-major visible-tile lists: rows r = h * nkt + kj (nkt = ceil(n/block_n)),
 * columns the query tiles qi in ascending order, flags as in cowa_plan. */
cowa_status cowa_plan_kv_size(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                              int32_t block_m, int32_t block_n, int64_t* nnz_out);
cowa_status cowa_plan_kv(const cowa_pattern* p, int32_t n, int32_t h_kv_local,
                         int32_t block_m, int32_t block_n,
                         int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t cap);

/* Workspace bytes of cowa_bwd for this pattern and shape (LSE and D per
 * query row, plus fp32 partial dK/dV of the key tiles holding sink keys,
 * whose work is split over several workgroups). */
cowa_status cowa_bwd_workspace_size(const cowa_pattern* p, int32_t B, int32_t H_q,
                                    int32_t H_kv_local, int32_t N, size_t* bytes);
cowa_status cowa_bwd(const cowa_pattern* p,
                     const int32_t* d_row_ptr, const int32_t* d_col, const uint8_t* d_flags,
                     int64_t nnz, int32_t block_m, int32_t block_n,
                     const int32_t* d_row_ptr_kv, const int32_t* d_col_kv,
                     const uint8_t* d_flags_kv, int64_t nnz_kv, int32_t block_m_kv,
                     int32_t block_n_kv,
                     const void* q, const void* k, const void* v, const void* o,
                     int32_t o_dtype, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int32_t g_dtype,
                     int32_t B, int32_t N, int32_t H_q, int32_t H_kv_local, int32_t d,
                     const int64_t strides[24], float softmax_scale,
                     void* workspace, size_t ws_bytes, void* stream);

/* Backward of the packed (varlen) prefill (cowa_fwd_varlen): the gradients of
 * n_seqs sequences of different lengths in one call, training on packed
 * batches with the same operator ("CoWindow Attention: Full Causal Coverage Is
 * a Collective Property", Abstract: one pattern in training and inference).
 * Sequence b is at token rows [cu_seqlens[b], cu_seqlens[b+1]) of q, o, dout,
 * dq [total_tokens, H_q, d] and k, v, dk, dv [total_tokens, H_kv_local, d];
 * positions restart at 0 in every sequence, and no sequence sees another's
 * tokens.
 *  cu_seqlens     device int32[n_seqs + 1], as in cowa_fwd_varlen (lengths
 *                 <= max_seqlen are not checked on the host: rows past
 *                 max_seqlen get no gradient)
 *  plans          cowa_plan and cowa_plan_kv for n = max_seqlen (one pair serves
 *                 every length)
 *  lse            forward LSE fp32 [H_q, total_tokens] (cowa_fwd_varlen's)
 *  strides        element strides (t, h) of q, k, v, o, dout, dq, dk, dv (16)
 *  workspace      cowa_bwd_workspace_size(p, n_seqs, H_q, H_kv_local,
 *                 max_seqlen) bytes, 256-byte aligned
 * Everything else, errors included, as in cowa_bwd; n_seqs, max_seqlen and
 * total_tokens must be >= 1 (COWA_ERR_INVALID_ARG otherwise). */
cowa_status cowa_bwd_varlen(const cowa_pattern* p,
                            const int32_t* d_row_ptr, const int32_t* d_col,
                            const uint8_t* d_flags, int64_t nnz, int32_t block_m,
                            int32_t block_n, const int32_t* d_row_ptr_kv,
                            const int32_t* d_col_kv, const uint8_t* d_flags_kv,
                            int64_t nnz_kv, int32_t block_m_kv, int32_t block_n_kv,
                            const void* q, const void* k, const void* v, const void* o,
                            int32_t o_dtype, const void* dout, const float* lse,
                            void* dq, void* dk, void* dv, int32_t g_dtype,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                            int32_t total_tokens, int32_t H_q, int32_t H_kv_local, int32_t d,
                            const int64_t strides[16], float softmax_scale,
                            void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COWA_H */
