// Host-side launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct ScoreShape {
  int L, H, G, d;
  int n_c;        // cached keys per head
  int n_in;       // query positions per head (n_prompt + n_c)
  float scale;    // logit temperature
};

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

// Gather of kept rows; see kv_compact.
hipError_t launch_compact(const uint16_t* k_ctx, const uint16_t* v_ctx,
                          const int64_t* offsets, const int32_t* idx,
                          uint16_t* k_out, uint16_t* v_out, int LH, int d,
                          int64_t n_c, int64_t total, hipStream_t stream);

}  // namespace kvq
