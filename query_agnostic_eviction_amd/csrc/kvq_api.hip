// C ABI of libkvq: argument checks on the host, then one enqueue per call on
// the caller's stream.  Declarations and contracts live in include/kvq.h.
#include <math.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KV_OK;
  g_last_hip = (int)e;
  return KV_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool valid_ratio(double r) { return r > 0.0 && r <= 1.0; }  // false for NaN

int64_t keep_count_of(int64_t n, double r) {
  double f = floor(r * (double)n);
  int64_t k = (int64_t)f;
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

// The logit scale of the scoring passes: 0 selects the model's temperature
// float32(1 / sqrt(d)); otherwise it must be positive with 1 / scale and the
// first running-max offset of pass 1, 1e30 * scale * log2(e), finite in fp32
// (both are formed by the passes).  Returns 0 for a rejected scale.
float resolve_scale(float scale, int d) {
  if (scale == 0.0f) return (float)(1.0 / sqrt((double)d));
  if (!(scale > 0.0f) || !isfinite(scale)) return 0.0f;
  const float c2 = scale * kvq::kLog2e;
  if (!isfinite(1.0e30f * c2) || !isfinite((float)(1.0 / (double)scale))) return 0.0f;
  return scale;
}

// Shared checks of the two scoring passes.
int check_score_args(int L, int H, int G, int d, int64_t n_c, int64_t n_prompt,
                     float scale, kvq::ScoreShape* out) {
  if (L < 1 || H < 1 || n_c < 1 || n_prompt < 0) return KV_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return KV_ERR_UNSUPPORTED;
  scale = resolve_scale(scale, d);
  if (scale == 0.0f) return KV_ERR_INVALID_ARG;
  if (G < 1 || G > 8) return KV_ERR_UNSUPPORTED;
  const int64_t n_in = n_prompt + n_c;
  if (n_c >= (int64_t)1 << 31 || (int64_t)G * n_in >= (int64_t)1 << 31)
    return KV_ERR_INVALID_ARG;
  if ((int64_t)L * H >= (int64_t)1 << 31) return KV_ERR_INVALID_ARG;
  *out = kvq::plain_shape(L, H, G, d, (int)n_c, (int)n_in, scale);
  return KV_OK;
}

// Chunked scoring (KVzip page section 3.4): chunk c of each (l, h) covers
// cached keys [c*chunk, c*chunk + m_c) with m_c = min(chunk, n_c - c*chunk)
// and has its own n_prompt + m_c query positions; per (l, h) the chunks'
// queries, new keys and lse are packed back to back (see kvq.h).  Full
// chunks run as one launch with a work item per (l, h, chunk); a shorter
// last chunk runs as a second launch with a work item per (l, h).
struct ChunkPlan {
  int n_launch;
  kvq::ScoreShape s[2];
};

int plan_chunks(int L, int H, int G, int d, int64_t n_c, int64_t n_prompt,
                int64_t chunk, float scale, ChunkPlan* plan) {
  if (chunk < 1) return KV_ERR_INVALID_ARG;
  kvq::ScoreShape base;
  int st = check_score_args(L, H, G, d, n_c, n_prompt, scale, &base);
  if (st != KV_OK) return st;
  const int64_t m = chunk < n_c ? chunk : n_c;
  const int64_t full = n_c / m, rem = n_c % m;
  const int64_t nchunks = full + (rem ? 1 : 0);
  const int64_t rows = nchunks * n_prompt + n_c;  // query positions per (l, h)
  if ((int64_t)G * (n_prompt + m) >= ((int64_t)1 << 31) ||
      (int64_t)L * H * full >= ((int64_t)1 << 31) || (int64_t)G * rows >= ((int64_t)1 << 40))
    return KV_ERR_INVALID_ARG;
  const long long dd = d, g = G;
  const long long slot = n_prompt + m;           // positions of a full chunk
  plan->n_launch = 0;
  if (full > 0) {
    kvq::ScoreShape& a = plan->s[plan->n_launch++];
    a = base;
    a.nheads = (int)((int64_t)L * H * full);
    a.inner = (int)full;
    a.n_c = (int)m;
    a.n_in = (int)slot;
    a.q = {0, g * rows * dd, g * slot * dd};
    a.k_new = {0, rows * dd, slot * dd};
    a.lse = {0, g * rows, g * slot};
    a.k_ctx = {0, n_c * dd, m * dd};
    a.scores = {0, n_c, m};
  }
  if (rem > 0) {
    kvq::ScoreShape& b = plan->s[plan->n_launch++];
    b = base;
    b.nheads = L * H;
    b.inner = 1;
    b.n_c = (int)rem;
    b.n_in = (int)(n_prompt + rem);
    b.q = {full * g * slot * dd, g * rows * dd, 0};
    b.k_new = {full * slot * dd, rows * dd, 0};
    b.lse = {full * g * slot, g * rows, 0};
    b.k_ctx = {full * m * dd, n_c * dd, 0};
    b.scores = {full * m, n_c, 0};
  }
  return KV_OK;
}

}  // namespace

extern "C" {

const char* kv_status_string(int status) {
  switch (status) {
    case KV_OK: return "KV_OK";
    case KV_ERR_INVALID_ARG: return "KV_ERR_INVALID_ARG";
    case KV_ERR_UNSUPPORTED: return "KV_ERR_UNSUPPORTED";
    case KV_ERR_ALIGNMENT: return "KV_ERR_ALIGNMENT";
    case KV_ERR_CAPACITY: return "KV_ERR_CAPACITY";
    case KV_ERR_HIP: return "KV_ERR_HIP";
    default: return "KV_ERR_UNKNOWN";
  }
}

int kv_last_hip_error(void) { return g_last_hip; }

int kv_keep_count(int64_t n, double keep_ratio, int64_t* k_out) {
  if (!k_out || n < 1 || !valid_ratio(keep_ratio)) return KV_ERR_INVALID_ARG;
  *k_out = keep_count_of(n, keep_ratio);
  return KV_OK;
}

int kvscore_lse(const void* q, const void* k_ctx, const void* k_new, float* lse,
                int L, int H, int G, int d, int64_t n_c, int64_t n_prompt,
                float scale, void* stream) {
  if (!q || !k_ctx || !k_new || !lse) return KV_ERR_INVALID_ARG;
  kvq::ScoreShape s;
  int st = check_score_args(L, H, G, d, n_c, n_prompt, scale, &s);
  if (st != KV_OK) return st;
  if (!aligned(q, 16) || !aligned(k_ctx, 16) || !aligned(k_new, 16) || !aligned(lse, 4))
    return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return hip_status(kvq::launch_lse(static_cast<const uint16_t*>(q),
                                    static_cast<const uint16_t*>(k_ctx),
                                    static_cast<const uint16_t*>(k_new), lse, s,
                                    static_cast<hipStream_t>(stream)));
}

int kvscore_colmax(const void* q, const void* k_ctx, const float* lse,
                   float* scores, int L, int H, int G, int d, int64_t n_c,
                   int64_t n_prompt, float scale, void* stream) {
  if (!q || !k_ctx || !lse || !scores) return KV_ERR_INVALID_ARG;
  kvq::ScoreShape s;
  int st = check_score_args(L, H, G, d, n_c, n_prompt, scale, &s);
  if (st != KV_OK) return st;
  if (!aligned(q, 16) || !aligned(k_ctx, 16) || !aligned(lse, 4) || !aligned(scores, 4))
    return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return hip_status(kvq::launch_colmax(static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k_ctx), lse,
                                       scores, s, static_cast<hipStream_t>(stream)));
}

int kv_chunk_layout(int64_t n_c, int64_t n_prompt, int64_t chunk,
                    int64_t* n_chunks, int64_t* rows_per_head) {
  if (!n_chunks || !rows_per_head || n_c < 1 || n_prompt < 0 || chunk < 1)
    return KV_ERR_INVALID_ARG;
  const int64_t m = chunk < n_c ? chunk : n_c;
  *n_chunks = (n_c + m - 1) / m;
  *rows_per_head = *n_chunks * n_prompt + n_c;
  return KV_OK;
}

int kvscore_chunked_lse(const void* q, const void* k_ctx, const void* k_new,
                        float* lse, int L, int H, int G, int d, int64_t n_c,
                        int64_t n_prompt, int64_t chunk, float scale,
                        void* stream) {
  if (!q || !k_ctx || !k_new || !lse) return KV_ERR_INVALID_ARG;
  ChunkPlan plan;
  int st = plan_chunks(L, H, G, d, n_c, n_prompt, chunk, scale, &plan);
  if (st != KV_OK) return st;
  if (!aligned(q, 16) || !aligned(k_ctx, 16) || !aligned(k_new, 16) || !aligned(lse, 4))
    return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  for (int i = 0; i < plan.n_launch; ++i) {
    st = hip_status(kvq::launch_lse(static_cast<const uint16_t*>(q),
                                    static_cast<const uint16_t*>(k_ctx),
                                    static_cast<const uint16_t*>(k_new), lse,
                                    plan.s[i], static_cast<hipStream_t>(stream)));
    if (st != KV_OK) return st;
  }
  return KV_OK;
}

int kvscore_chunked_colmax(const void* q, const void* k_ctx, const float* lse,
                           float* scores, int L, int H, int G, int d,
                           int64_t n_c, int64_t n_prompt, int64_t chunk,
                           float scale, void* stream) {
  if (!q || !k_ctx || !lse || !scores) return KV_ERR_INVALID_ARG;
  ChunkPlan plan;
  int st = plan_chunks(L, H, G, d, n_c, n_prompt, chunk, scale, &plan);
  if (st != KV_OK) return st;
  if (!aligned(q, 16) || !aligned(k_ctx, 16) || !aligned(lse, 4) || !aligned(scores, 4))
    return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  for (int i = 0; i < plan.n_launch; ++i) {
    st = hip_status(kvq::launch_colmax(static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k_ctx), lse,
                                       scores, plan.s[i],
                                       static_cast<hipStream_t>(stream)));
    if (st != KV_OK) return st;
  }
  return KV_OK;
}

int kv_topk_total(int L, int H, int64_t n_c, double keep_ratio, int mode,
                  int64_t* total_out) {
  if (!total_out || L < 1 || H < 1 || n_c < 1 || !valid_ratio(keep_ratio))
    return KV_ERR_INVALID_ARG;
  if (mode < 0 || mode > 2) return KV_ERR_UNSUPPORTED;
  if ((int64_t)H * n_c >= (int64_t)1 << 31 || (int64_t)L * H >= (int64_t)1 << 31)
    return KV_ERR_INVALID_ARG;
  // mode 2 counts per workgroup in 32 bits: at most 2^40 scores (4 TiB)
  if (mode == 2 && (int64_t)L * H * n_c >= (int64_t)1 << 40) return KV_ERR_INVALID_ARG;
  if (mode == 0)
    *total_out = (int64_t)L * H * keep_count_of(n_c, keep_ratio);
  else if (mode == 1)
    *total_out = (int64_t)L * keep_count_of((int64_t)H * n_c, keep_ratio);
  else
    *total_out = keep_count_of((int64_t)L * H * n_c, keep_ratio);
  return KV_OK;
}

size_t kv_topk_workspace_bytes(int L, int H, int64_t n_c, int mode) {
  if (mode != 2 || L < 1 || H < 1 || n_c < 1) return 0;
  return kvq::global_select_workspace((int64_t)L * H * n_c);
}

int kv_topk_select(const float* scores, int L, int H, int64_t n_c,
                   double keep_ratio, int mode, int64_t* offsets, int32_t* idx,
                   int64_t capacity, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!scores || !offsets || !idx) return KV_ERR_INVALID_ARG;
  int64_t total = 0;
  int st = kv_topk_total(L, H, n_c, keep_ratio, mode, &total);
  if (st != KV_OK) return st;
  if (!aligned(scores, 4) || !aligned(offsets, 8) || !aligned(idx, 4))
    return KV_ERR_ALIGNMENT;
  const size_t ws_need = kv_topk_workspace_bytes(L, H, n_c, mode);
  if (capacity < total || workspace_bytes < ws_need) return KV_ERR_CAPACITY;
  if (ws_need && !workspace) return KV_ERR_INVALID_ARG;
  if (ws_need && !aligned(workspace, 256)) return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  if (mode == 2)
    return hip_status(kvq::launch_global_topk(scores, (int64_t)L * H * n_c, (int)n_c, L * H,
                                              total, offsets, idx, workspace,
                                              static_cast<hipStream_t>(stream)));
  const int64_t k = mode == 0 ? keep_count_of(n_c, keep_ratio)
                              : keep_count_of((int64_t)H * n_c, keep_ratio);
  return hip_status(kvq::launch_topk(scores, L, H, (int)n_c, mode, k, offsets,
                                     idx, static_cast<hipStream_t>(stream)));
}

int kv_topk_select_noalloc(const float* scores, int L, int H, int64_t n_c,
                           double keep_ratio, int mode, int64_t* offsets,
                           int32_t* idx, int64_t capacity, void* stream) {
  if (!scores || !offsets || !idx) return KV_ERR_INVALID_ARG;
  int64_t total = 0;
  int st = kv_topk_total(L, H, n_c, keep_ratio, mode, &total);
  if (st != KV_OK) return st;
  if (!aligned(scores, 4) || !aligned(offsets, 8) || !aligned(idx, 4))
    return KV_ERR_ALIGNMENT;
  if (capacity < total) return KV_ERR_CAPACITY;
  const size_t ws_need = kv_topk_workspace_bytes(L, H, n_c, mode);
  if (ws_need > kvq::kNoAllocScratchBytes) return KV_ERR_CAPACITY;
  if (mode != 2)  // no scratch: the same launch as kv_topk_select
    return kv_topk_select(scores, L, H, n_c, keep_ratio, mode, offsets, idx, capacity,
                          nullptr, 0, stream);
  void* ws = nullptr;
  st = hip_status(kvq::noalloc_scratch(&ws));
  if (st != KV_OK) return st;
  (void)hipGetLastError();
  return hip_status(kvq::launch_global_topk(scores, (int64_t)L * H * n_c, (int)n_c, L * H,
                                            total, offsets, idx, ws,
                                            static_cast<hipStream_t>(stream)));
}

int kv_head_scores(const float* scores, int L, int H, int64_t n_c,
                   float* head_scores, void* stream) {
  if (!scores || !head_scores || L < 1 || H < 1 || n_c < 1) return KV_ERR_INVALID_ARG;
  if ((int64_t)L * H >= (int64_t)1 << 31 || (int64_t)H * n_c >= (int64_t)1 << 31)
    return KV_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(head_scores, 4)) return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return hip_status(kvq::launch_head_max(scores, L * H, (int)n_c, head_scores,
                                         static_cast<hipStream_t>(stream)));
}

int kv_compact(const void* k_ctx, const void* v_ctx, const int64_t* offsets,
               const int32_t* idx, void* k_out, void* v_out, int L, int H,
               int d, int64_t n_c, int64_t total, void* stream) {
  if (!k_ctx || !v_ctx || !offsets) return KV_ERR_INVALID_ARG;
  // an empty kept set has empty (possibly null) idx and outputs
  if (total > 0 && (!idx || !k_out || !v_out)) return KV_ERR_INVALID_ARG;
  if (L < 1 || H < 1 || n_c < 1 || total < 0) return KV_ERR_INVALID_ARG;
  if ((int64_t)L * H >= (int64_t)1 << 31 || n_c >= (int64_t)1 << 31) return KV_ERR_INVALID_ARG;
  if (total > (int64_t)L * H * n_c) return KV_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return KV_ERR_UNSUPPORTED;
  if (!aligned(k_ctx, 16) || !aligned(v_ctx, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || !aligned(offsets, 8) || !aligned(idx, 4))
    return KV_ERR_ALIGNMENT;
  if (total == 0) return KV_OK;
  (void)hipGetLastError();
  return hip_status(kvq::launch_compact(
      static_cast<const uint16_t*>(k_ctx), static_cast<const uint16_t*>(v_ctx),
      offsets, idx, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out),
      L * H, d, n_c, total, 0, static_cast<hipStream_t>(stream)));
}

int kv_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || bytes % 16 != 0) return KV_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return KV_ERR_ALIGNMENT;
  if (bytes == 0) return KV_OK;
  (void)hipGetLastError();
  return hip_status(kvq::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int kv_epi_deltas(const void* h, int n_layers, int64_t n, int D, float* g, void* stream) {
  if (!h || !g || n_layers < 1 || n < 1) return KV_ERR_INVALID_ARG;
  if (D < 8 || D > 8192 || D % 8 != 0) return KV_ERR_UNSUPPORTED;
  // one workgroup per run of 16 rows of a layer: the grid must stay < 2^31
  if (n >= (int64_t)1 << 36 || (int64_t)n_layers * ((n + 15) / 16) >= (int64_t)1 << 31)
    return KV_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(g, 4)) return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return hip_status(kvq::launch_epi_deltas(static_cast<const uint16_t*>(h), n_layers, n, D, g,
                                           static_cast<hipStream_t>(stream)));
}

int kv_epi_scores(const float* g, int n_a, int n_b, int64_t n, int window, double eps,
                  int detrend, float* scores, void* stream) {
  if (!g || !scores || n_a < 1 || n_b < 1 || n < 1 || window < 1) return KV_ERR_INVALID_ARG;
  if (!(eps > 0.0) || !isfinite(eps) || (detrend != 0 && detrend != 1))
    return KV_ERR_INVALID_ARG;
  if (window > 1024) return KV_ERR_UNSUPPORTED;
  if ((int64_t)n_a + n_b > 4096 || n >= (int64_t)1 << 36) return KV_ERR_INVALID_ARG;
  if (!aligned(g, 4) || !aligned(scores, 4)) return KV_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return hip_status(kvq::launch_epi_scores(g, n_a, n_b, n, window, eps, detrend, scores,
                                           static_cast<hipStream_t>(stream)));
}

size_t kv_select_tokens_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  return kvq::global_select_workspace(n);
}

int kv_select_tokens(const float* scores, int64_t n, int64_t k, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !idx || !workspace || n < 1 || k < 1 || k > n) return KV_ERR_INVALID_ARG;
  if (n >= (int64_t)1 << 31) return KV_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(idx, 4) || !aligned(workspace, 256))
    return KV_ERR_ALIGNMENT;
  if (workspace_bytes < kv_select_tokens_workspace_bytes(n)) return KV_ERR_CAPACITY;
  (void)hipGetLastError();
  return hip_status(kvq::launch_select_tokens_grid(scores, n, k, idx, workspace,
                                                   static_cast<hipStream_t>(stream)));
}

int kv_compact_tokens(const void* k_cache, const void* v_cache, const int32_t* idx,
                      void* k_out, void* v_out, int L, int H, int d, int64_t n, int64_t k,
                      void* stream) {
  if (!k_cache || !v_cache) return KV_ERR_INVALID_ARG;
  if (k > 0 && (!idx || !k_out || !v_out)) return KV_ERR_INVALID_ARG;
  if (L < 1 || H < 1 || n < 1 || k < 0 || k > n) return KV_ERR_INVALID_ARG;
  if ((int64_t)L * H >= (int64_t)1 << 31 || n >= (int64_t)1 << 31) return KV_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return KV_ERR_UNSUPPORTED;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || !aligned(idx, 4))
    return KV_ERR_ALIGNMENT;
  if (k == 0) return KV_OK;
  (void)hipGetLastError();
  return hip_status(kvq::launch_compact(
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), nullptr,
      idx, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), L * H, d, n,
      (int64_t)L * H * k, k, static_cast<hipStream_t>(stream)));
}

int kv_merge_compact(const void* k_ctx, const void* v_ctx, const int64_t* offsets,
                     const int32_t* idx, const int64_t* src_offsets, const int32_t* src_idx,
                     void* k_out, void* v_out, float* gate, float* mass, int L, int H, int d,
                     int64_t n_c, int64_t total, int64_t n_src, void* stream) {
  if (!k_ctx || !v_ctx || !offsets || !src_offsets) return KV_ERR_INVALID_ARG;
  if (total > 0 && (!idx || !k_out || !v_out)) return KV_ERR_INVALID_ARG;
  if (n_src > 0 && !src_idx) return KV_ERR_INVALID_ARG;
  if (L < 1 || H < 1 || n_c < 1 || total < 0 || n_src < 0) return KV_ERR_INVALID_ARG;
  if ((int64_t)L * H >= (int64_t)1 << 31 || n_c >= (int64_t)1 << 31) return KV_ERR_INVALID_ARG;
  if (total > (int64_t)L * H * n_c) return KV_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return KV_ERR_UNSUPPORTED;
  if (!aligned(k_ctx, 16) || !aligned(v_ctx, 16) || !aligned(k_out, 16) ||
      !aligned(v_out, 16) || !aligned(offsets, 8) || !aligned(idx, 4) ||
      !aligned(src_offsets, 8) || !aligned(src_idx, 4) || !aligned(gate, 4) ||
      !aligned(mass, 4))
    return KV_ERR_ALIGNMENT;
  if (total == 0) return KV_OK;
  (void)hipGetLastError();
  return hip_status(kvq::launch_merge(
      static_cast<const uint16_t*>(k_ctx), static_cast<const uint16_t*>(v_ctx), offsets, idx,
      src_offsets, src_idx, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), gate,
      mass, L * H, d, n_c, total, n_src, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
