/*
 * kvq.h - query-agnostic KV cache scoring, selection and compaction on AMD
 * Instinct MI355X (gfx950).  C ABI; every entry point takes plain pointers and
 * sizes and enqueues work on the caller's HIP stream.
 *
 * The computation is the KVzip importance score (page "KVzip: Query-Agnostic
 * KV Cache Compression with Context Reconstruction"):
 *   section 2.1  - a prefilled context of n_c tokens caches L x H x n_c KV
 *                  pairs (KV_c) in a model with L layers and H KV heads, each
 *                  KV head serving a group of G query heads; the goal is a
 *                  subset KV_p of KV_c;
 *   section 3.2  - a teacher-forced pass over the repeat prompt (n_prompt
 *                  tokens) followed by the context gives, per (l, h), grouped
 *                  queries Q (G x n_in x d, n_in = n_prompt + n_c) and keys
 *                  K = [cached keys; new keys] ((n_c + n_in) x d);
 *                  A = Softmax(Q K^T); the score of cached key j is the max of
 *                  A[g, i, j] over all g and all n_in rows i;
 *   section 4.1  - keep the r% highest-scoring pairs.
 *
 * Readings fixed by this library where the page is silent:
 *   - logits are scale * <q, k> with the model's attention temperature
 *     scale = 1 / sqrt(d); the scoring calls take it as an argument, and
 *     scale = 0 selects that default, float32(1 / sqrt(d)), formed here;
 *   - row i (0-based) of the pass sees all n_c cached keys and new keys
 *     0..i, its own included; every one of the n_in rows counts;
 *   - the softmax is normalised over every key a row sees, then sliced;
 *   - the kept count is k = clamp(floor(r * n), 1, n) (the floor rule of the
 *     SelKV page, "Selective KV cache merging", section 3.1); equal scores
 *     are broken toward the lower index; kept indices come out ascending.
 *
 * Layouts (all row-major, contiguous, no padding):
 *   q       bf16  [L][H][G][n_in][d]   query head h*G + g serves KV head h
 *   k_ctx   bf16  [L][H][n_c][d]       cached keys (KV_c)
 *   k_new   bf16  [L][H][n_in][d]      keys of the repeat pass
 *   v_ctx   bf16  [L][H][n_c][d]       cached values
 *   lse     fp32  [L][H][G][n_in]      natural-log row normaliser
 *   scores  fp32  [L][H][n_c]          score of every cached key, in [0, 1]
 *   offsets int64 [L*H + 1]            CSR offsets of the kept sets
 *   idx     int32 [total]              kept positions j in [0, n_c)
 *   k_out, v_out bf16 [total][d]       kept rows, grouped by (l, h)
 *
 * Conventions shared by every entry point:
 *   - Device pointers are owned by the caller; the library never allocates,
 *     frees or retains them.  bf16 tensors must be 16-byte aligned, fp32 and
 *     int32 ones 4-byte aligned, int64 ones 8-byte aligned.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error nothing is written and a negative status is returned.
 *   - Work is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  A launch failure returns KV_ERR_HIP and records the HIP error
 *     for kv_last_hip_error(); faults during execution surface at the
 *     caller's next synchronisation.
 *   - Inputs must be finite, and so must the logits scale * <q, k> that the
 *     scoring passes form in fp32 (any bf16 inputs of model scale qualify).
 *     Calls are reentrant; calls that write the same buffers must not
 *     overlap.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define KV_OK                0
#define KV_ERR_INVALID_ARG  -1  /* null pointer, non-positive size, ratio out of (0,1], size overflow */
#define KV_ERR_UNSUPPORTED  -2  /* d not in {64, 128, 256}, G not in [1, 8], mode not in {0, 1, 2} */
#define KV_ERR_ALIGNMENT    -3  /* a pointer breaks the alignment rule above */
#define KV_ERR_CAPACITY     -4  /* idx capacity or workspace too small */
#define KV_ERR_HIP          -5  /* a HIP runtime call or launch failed */

/* Human-readable name of a status code (static storage; never NULL). */
const char* kv_status_string(int status);

/* hipError_t of the most recent KV_ERR_HIP on the calling thread (0 if none). */
int kv_last_hip_error(void);

/* Kept count for a set of n scores at keep ratio r (KVzip section 4.1 budget,
 * SelKV section 3.1 floor rule): *k_out = clamp(floor(r * n), 1, n), computed
 * in IEEE double.  Pure host function.  KV_ERR_INVALID_ARG if n < 1, k_out is
 * NULL or r is not in (0, 1]. */
int kv_keep_count(int64_t n, double keep_ratio, int64_t* k_out);

/* Pass 1 (KVzip section 3.2, the softmax of A = Softmax(Q K^T)): for every
 * (l, h, g, i) writes
 *   lse[l][h][g][i] = ln sum_{j seen by row i} exp(scale * <q_{g,i}, k_j>)
 * over the n_c cached keys and new keys 0..i.  The attention matrix is never
 * stored.  Requires L, H >= 1, 1 <= G <= 8, d in {64, 128, 256}, n_c >= 1,
 * n_prompt >= 0, G * (n_prompt + n_c) < 2^31, and scale = 0 (the default
 * float32(1 / sqrt(d))) or a positive scale for which both 1 / scale and
 * 1e30 * scale * log2(e) are finite in fp32 (about 3e-39 <= scale <= 2.3e8;
 * the passes form both).  KV_ERR_INVALID_ARG otherwise. */
int kvscore_lse(const void* q, const void* k_ctx, const void* k_new, float* lse,
                int L, int H, int G, int d, int64_t n_c, int64_t n_prompt,
                float scale, void* stream);

/* Pass 2 (KVzip section 3.2, the sliced matrix and its max): for every cached
 * key writes
 *   scores[l][h][j] = max_{g, i} exp(scale * <q_{g,i}, k_j> - lse[l][h][g][i])
 * for j < n_c, i.e. the largest softmax probability key j receives.  lse must
 * hold pass 1's output for the same inputs.  Every score is written (no
 * pre-zeroed buffer is needed); the result does not depend on scheduling.
 * Same requirements as kvscore_lse. */
int kvscore_colmax(const void* q, const void* k_ctx, const float* lse,
                   float* scores, int L, int H, int G, int d, int64_t n_c,
                   int64_t n_prompt, float scale, void* stream);

/* Chunked scoring (KVzip section 3.4, chunk-based scoring): the context is
 * split into chunks of `chunk` tokens (the last one shorter when chunk does
 * not divide n_c); chunk c of every (l, h) is scored on its own, from a
 * repeat pass over the prompt and that chunk only: m_c = min(chunk,
 * n_c - c*chunk) cached keys [c*chunk, c*chunk + m_c) and n_in_c = n_prompt +
 * m_c new keys, an n_in_c x (m_c + n_in_c) attention per query head, causal
 * over the new keys, normalised over those keys only.  Each chunk's scores
 * land at its keys' positions in the usual scores[l][h][n_c].
 *
 * Layouts (per (l, h), chunks packed back to back in chunk order):
 *   q     bf16 [L][H][rows * G][d]   chunk c is a [G][n_in_c][d] block
 *   k_new bf16 [L][H][rows][d]       chunk c is a [n_in_c][d] block
 *   lse   fp32 [L][H][rows * G]      chunk c is a [G][n_in_c] block
 *   k_ctx, scores as for the unchunked calls
 * where rows = n_chunks * n_prompt + n_c (kv_chunk_layout).  chunk >= n_c is
 * exactly the unchunked computation.  Same requirements and errors as the
 * unchunked calls, plus chunk >= 1 and G * (n_prompt + min(chunk, n_c)) < 2^31. */
int kv_chunk_layout(int64_t n_c, int64_t n_prompt, int64_t chunk,
                    int64_t* n_chunks, int64_t* rows_per_head);
int kvscore_chunked_lse(const void* q, const void* k_ctx, const void* k_new,
                        float* lse, int L, int H, int G, int d, int64_t n_c,
                        int64_t n_prompt, int64_t chunk, float scale,
                        void* stream);
int kvscore_chunked_colmax(const void* q, const void* k_ctx, const float* lse,
                           float* scores, int L, int H, int G, int d,
                           int64_t n_c, int64_t n_prompt, int64_t chunk,
                           float scale, void* stream);

/* Total kept count for kv_topk_select: L*H*k (mode 0, k = keep count of n_c),
 * L*k_L (mode 1, k_L = keep count of H*n_c) or k_M (mode 2, keep count of
 * L*H*n_c).  Pure host function.  Limits: L*H < 2^31, H*n_c < 2^31 and, in
 * mode 2, L*H*n_c < 2^40 (KV_ERR_INVALID_ARG otherwise). */
int kv_topk_total(int L, int H, int64_t n_c, double keep_ratio, int mode,
                  int64_t* total_out);

/* Device scratch bytes kv_topk_select needs for these sizes: 0 for modes 0
 * and 1 (NULL workspace accepted), about 16 KiB + 16 B per 4096 scores (or
 * per 1/1024 of the scores, whichever is more) for mode 2.  The workspace is owned by the caller, must be 256-byte aligned,
 * need not be initialised, and must not be shared by overlapping calls. */
size_t kv_topk_workspace_bytes(int L, int H, int64_t n_c, int mode);

/* Selection (KVzip section 4.1): keeps the highest scores.
 *   mode 0: per (l, h), the k = clamp(floor(r * n_c), 1, n_c) largest;
 *   mode 1: per layer l, the k_L = clamp(floor(r * H * n_c), 1, H * n_c)
 *           largest of the layer's H * n_c scores (a non-uniform per-head
 *           budget); heads receive different counts;
 *   mode 2: the k_M = clamp(floor(r * L * H * n_c), 1, L * H * n_c) largest
 *           of all the model's scores (one budget across every head of every
 *           layer); layers and heads receive different counts.
 * Equal scores go to the lower index (j; h * n_c + j in mode 1; (l * H + h) *
 * n_c + j in mode 2).  Mode 2 runs as a sequence of grid-wide launches and
 * needs the workspace of kv_topk_workspace_bytes.  Writes
 * offsets[L*H + 1] (offsets[l*H + h] = first kept row of that head) and the
 * kept positions j into idx, ascending within each head.  scores must be
 * non-negative (they are ordered by their IEEE bit pattern, with -0.0 read
 * as +0.0).  capacity is the
 * length of idx; KV_ERR_CAPACITY if it is below the total (kv_topk_total). */
int kv_topk_select(const float* scores, int L, int H, int64_t n_c,
                   double keep_ratio, int mode, int64_t* offsets, int32_t* idx,
                   int64_t capacity, void* workspace, size_t workspace_bytes,
                   void* stream);

/* kv_topk_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * same arguments, results and errors, without the workspace.  Mode 2 keeps
 * its grid-wide state in a file-scope device array of 48 KiB (one per GPU,
 * held until the process ends; every valid size needs at most ~33 KiB, and a
 * larger need returns KV_ERR_CAPACITY).  Its address is looked up once per
 * device on the first call there (hipGetSymbolAddress; a failure returns
 * KV_ERR_HIP); the call itself allocates nothing.  Every call on one GPU
 * shares that array, so calls that overlap on one GPU (for instance on two
 * streams) race; calls ordered on one stream do not.  Modes 0 and 1 use no
 * scratch. */
int kv_topk_select_noalloc(const float* scores, int L, int H, int64_t n_c,
                           double keep_ratio, int mode, int64_t* offsets,
                           int32_t* idx, int64_t capacity, void* stream);

/* Head-level static score (KVzip section 4.2, context-independent
 * eviction): head_scores[l][h] = max_j scores[l][h][j], the largest pair
 * score of each head along the sequence, as fp32 [L][H].  Exact (a max of
 * the inputs, no rounding).  The heads can then be ranked by running
 * kv_topk_select on head_scores viewed as [1][1][L*H]. */
int kv_head_scores(const float* scores, int L, int H, int64_t n_c,
                   float* head_scores, void* stream);

/* Compaction (KVzip section 2.1, KV_p as a subset of KV_c): for every head
 * (l, h) and every t in [offsets[l*H+h], offsets[l*H+h+1]) copies
 *   k_out[t] = k_ctx[l][h][idx[t]],  v_out[t] = v_ctx[l][h][idx[t]]
 * bit for bit.  total = offsets[L*H] (known on the host from kv_topk_total),
 * or any larger count of rows that idx, k_out and v_out hold: rows from
 * offsets[L*H] on are then neither read nor written.
 * offsets must be non-decreasing with offsets[0] = 0; a row whose index falls
 * outside [0, n_c) is written as zeros instead of being read.  d in
 * {64, 128, 256}; L*H < 2^31, n_c < 2^31, 0 <= total <= L*H*n_c.  With
 * total = 0 nothing is enqueued and idx, k_out and v_out may be NULL. */
int kv_compact(const void* k_ctx, const void* v_ctx, const int64_t* offsets,
               const int32_t* idx, void* k_out, void* v_out, int L, int H,
               int d, int64_t n_c, int64_t total, void* stream);

/* Plain device-to-device copy of `bytes` (a multiple of 16; src and dst
 * 16-byte aligned, not overlapping), with the compaction's 16-byte
 * non-temporal loads and stores and four loads in flight per thread.  Not a
 * step of the method: the streaming reference that the compaction's HBM rate
 * is read against. */
int kv_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Gated merge instead of drop (page "Selective KV cache merging", section
 * 1: the soft cosine gate).  For kept row t (head lh with offsets[lh] <= t <
 * offsets[lh+1], position idx[t]) and every routed position j listed in
 * src_idx[src_offsets[t] .. src_offsets[t+1]) (positions of the same head):
 *   g_j  = max(<v_j, v_t> / (|v_j| |v_t|), 0)   (0 if a norm is 0 or j is
 *          outside [0, n_c))
 *   k_out[t] = (k_t + sum_j g_j k_j) / (1 + sum_j g_j), v_out likewise,
 * summed in fp32 in list order and rounded to bf16 (nearest-even);
 * gate[s] = g of entry s (n_src floats) and mass[t] = sum_j g_j (total
 * floats), each skipped when its pointer is NULL.  The page stops before
 * its routing and merge sections, so the routing is the caller's (any rule
 * producing the lists) and the merge is read as this weighted mean; with
 * every list empty the call equals kv_compact.  src_offsets int64 [total+1]
 * non-decreasing from 0 to n_src (ranges are clamped to [0, n_src)); kept
 * rows with an index outside [0, n_c) come out as zeros.  d in
 * {64, 128, 256}.  With total = 0 nothing is enqueued and idx, k_out and
 * v_out may be NULL (src_offsets still holds its one entry). */
int kv_merge_compact(const void* k_ctx, const void* v_ctx, const int64_t* offsets,
                     const int32_t* idx, const int64_t* src_offsets,
                     const int32_t* src_idx, void* k_out, void* v_out, float* gate,
                     float* mass, int L, int H, int d, int64_t n_c, int64_t total,
                     int64_t n_src, void* stream);

/* ------------------------------------------------------------------------
 * Attention-free token score (page "EpiKV", section 3.2, equations 1-3) and
 * token-level eviction under a budget of K tokens (section 3.1).  No
 * attention matrix is involved: the score reads hidden states only.
 *
 * Readings fixed by this library where the page is silent:
 *   - g(0) is undefined (no predecessor): stored as 0, in no window, and
 *     position 0 scores 0;
 *   - the window of position t >= 1 is the defined positions
 *     max(1, t - w + 1) .. t, the current one included;
 *   - sigma is the population standard deviation; eps is an argument;
 *   - a band is a set of layers whose statistics are averaged (the page's
 *     equations use one layer per band: 10 and 21);
 *   - the same K positions are kept in every layer and KV head.
 *
 * Layouts:
 *   h        bf16 [n_layers][n][D]     hidden states, band A's layers first
 *   g        fp32 [n_layers][n]        hidden-state change norms
 *   scores   fp32 [n]                  token scores (signed)
 *   idx      int32 [K]                 kept positions, ascending
 *   k_cache, v_cache bf16 [L][H][n][d]; k_out, v_out bf16 [L][H][K][d]
 * ------------------------------------------------------------------------ */

/* Equation 1: g[l][t] = || h[l][t] - h[l][t-1] ||_2 for t >= 1, g[l][0] = 0.
 * Differences of the bf16 inputs are formed and squared in fp32 and summed
 * in fp32 (relative error below 1e-5 for D <= 8192).  Requires n_layers,
 * n >= 1 and D a multiple of 8 in [8, 8192] (else KV_ERR_UNSUPPORTED); h
 * 16-byte aligned. */
int kv_epi_deltas(const void* h, int n_layers, int64_t n, int D, float* g,
                  void* stream);

/* Equations 2 and 3: for t >= 1, with W(t) the window above,
 *   detrend = 1:  stat_l(t) = (g_l(t) - mean_W g_l) / (std_W g_l + eps)
 *   detrend = 0:  stat_l(t) = mean_W g_l
 *   scores[t] = mean over band A (rows 0..n_a-1 of g) of stat_l(t)
 *             - mean over band B (rows n_a..n_a+n_b-1) of stat_l(t),
 * scores[0] = 0.  Window statistics in fp64, result rounded to fp32.
 * Requires n_a, n_b >= 1, 1 <= window <= 1024 (above: KV_ERR_UNSUPPORTED),
 * eps > 0 and finite, detrend in {0, 1}. */
int kv_epi_scores(const float* g, int n_a, int n_b, int64_t n, int window,
                  double eps, int detrend, float* scores, void* stream);

/* Device scratch bytes kv_select_tokens needs for n scores (about 16 KiB
 * plus 16 B per 4096 scores). */
size_t kv_select_tokens_workspace_bytes(int64_t n);

/* Budget of section 3.1: the k largest of n finite signed scores, ties (and
 * -0.0 vs +0.0) to the lower position, written to idx[0..k) ascending.  Runs
 * as a grid-wide radix select (six stream-ordered launches) in the caller's
 * workspace: 256-byte aligned, uninitialised, at least
 * kv_select_tokens_workspace_bytes(n) bytes (else KV_ERR_CAPACITY), not
 * shared by overlapping calls.  Requires 1 <= k <= n < 2^31. */
int kv_select_tokens(const float* scores, int64_t n, int64_t k, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Token-level compaction: k_out[l][h][t] = k_cache[l][h][idx[t]] and the
 * same for v, bit for bit, for t < k, every (l, h).  An index outside
 * [0, n) gives a zero row.  0 <= k <= n; d in {64, 128, 256}.  With k = 0
 * nothing is enqueued and idx, k_out and v_out may be NULL. */
int kv_compact_tokens(const void* k_cache, const void* v_cache,
                      const int32_t* idx, void* k_out, void* v_out, int L,
                      int H, int d, int64_t n, int64_t k, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
