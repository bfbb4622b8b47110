// Host-side launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// log2(e): the scoring passes take exp as exp2 with the logit scale folded in
constexpr float kLog2e = 1.4426950408889634f;

// Where one tensor of work item ("head") u lives, as an element offset:
//   off0 + (u / inner) * outer + (u % inner) * step
// An unchunked call has one work item per (layer, KV head) and inner = 1;
// chunked scoring has one per (layer, KV head, chunk) with inner = chunks.
struct TensorMap {
  long long off0, outer, step;
};

__host__ __device__ inline long long map_offset(const TensorMap& m, int u, int inner) {
  return m.off0 + (long long)(u / inner) * m.outer + (long long)(u % inner) * m.step;
}

struct ScoreShape {
  int nheads;     // work items of this launch
  int inner;      // work items per (layer, KV head)
  int G, d;
  int n_c;        // cached keys per work item
  int n_in;       // query positions per work item (n_prompt + its keys)
  float scale;    // logit temperature
  TensorMap q, k_new, lse, k_ctx, scores;
};

// The plain per-(layer, KV head) mapping of the layouts in kvq.h.
inline ScoreShape plain_shape(int L, int H, int G, int d, int n_c, int n_in, float scale) {
  ScoreShape s;
  s.nheads = L * H;
  s.inner = 1;
  s.G = G;
  s.d = d;
  s.n_c = n_c;
  s.n_in = n_in;
  s.scale = scale;
  s.q = {0, (long long)G * n_in * d, 0};
  s.k_new = {0, (long long)n_in * d, 0};
  s.lse = {0, (long long)G * n_in, 0};
  s.k_ctx = {0, (long long)n_c * d, 0};
  s.scores = {0, (long long)n_c, 0};
  return s;
}

// Pass 1: row log-sum-exp over cached keys and causal new keys.
hipError_t launch_lse(const uint16_t* q, const uint16_t* k_ctx,
                      const uint16_t* k_new, float* lse, const ScoreShape& s,
                      hipStream_t stream);

// Pass 2: per cached key, max over rows of exp(scale * q.k - lse).
hipError_t launch_colmax(const uint16_t* q, const uint16_t* k_ctx,
                         const float* lse, float* scores, const ScoreShape& s,
                         hipStream_t stream);

// Top-k over segments of scores; see kv_topk_select.
hipError_t launch_topk(const float* scores, int L, int H, int n_c, int mode,
                       int64_t k_per_segment, int64_t* offsets, int32_t* idx,
                       hipStream_t stream);

// Model-wide top-k over n scores (heads of n_c each) through the workspace.
long long global_select_per_block(long long n);
size_t global_select_workspace(long long n);
hipError_t launch_global_topk(const float* scores, long long n, int n_c, int nheads,
                              long long k, int64_t* offsets, int32_t* idx,
                              void* workspace, hipStream_t stream);

// Size of the file-scope device array behind kv_topk_select_noalloc, and the
// current device's address of it (looked up once per device).
constexpr size_t kNoAllocScratchBytes = 48 * 1024;
hipError_t noalloc_scratch(void** ptr);

// Max of each head's scores.
hipError_t launch_head_max(const float* scores, int nheads, int n_c, float* out,
                           hipStream_t stream);

// Gather of kept rows; see kv_compact.
// shared_k > 0: one kept set of shared_k positions for every head, no offsets.
hipError_t launch_compact(const uint16_t* k_ctx, const uint16_t* v_ctx,
                          const int64_t* offsets, const int32_t* idx,
                          uint16_t* k_out, uint16_t* v_out, int LH, int d,
                          int64_t n_c, int64_t total, int64_t shared_k,
                          hipStream_t stream);

// Plain streaming copy of `bytes` (a multiple of 16); see kv_copy.
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

// Top-k of n signed finite floats (ties to the lower index), ascending, by
// the grid-wide select (workspace of global_select_workspace(n) bytes).
hipError_t launch_select_tokens_grid(const float* scores, long long n, long long k,
                                     int32_t* idx, void* workspace, hipStream_t stream);

// Gated merge of routed tokens into kept rows (SelKV soft cosine gate).
hipError_t launch_merge(const uint16_t* k_ctx, const uint16_t* v_ctx, const int64_t* offsets,
                        const int32_t* idx, const int64_t* src_offsets, const int32_t* src_idx,
                        uint16_t* k_out, uint16_t* v_out, float* gate, float* mass, int LH,
                        int d, int64_t n_c, int64_t total, int64_t n_src, hipStream_t stream);

// EpiKV token score: hidden-state change norms, then band statistics.
hipError_t launch_epi_deltas(const uint16_t* h, int n_layers, int64_t n, int D, float* g,
                             hipStream_t stream);
hipError_t launch_epi_scores(const float* g, int n_a, int n_b, int64_t n, int w, double eps,
                             int detrend, float* scores, hipStream_t stream);

}  // namespace kvq
