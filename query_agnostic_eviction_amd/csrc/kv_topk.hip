// Selection of the kept KV pairs (KVzip page, "KVzip: Query-Agnostic KV
// Cache Compression with Context Reconstruction", section 4.1: keep the r%
// highest-scoring pairs; kept count floor(r * n) as in the SelKV page,
// section 3.1, clamped to [1, n]).
//
// One workgroup of 1024 threads per segment: a segment is one (l, h) row of
// n_c scores (mode 0) or one layer's H * n_c scores (mode 1, a budget shared
// by the layer's heads).  Scores are non-negative floats, so their IEEE bit
// patterns order like the values and can be radix-selected as uint32:
//  1. three histogram passes (11, 11, 10 bits, LDS atomics) fix the exact bit
//     pattern T of the k-th largest score and how many scores equal to T must
//     still be taken;
//  2. one ordered pass keeps every score above T and the lowest-index scores
//     equal to T, writing kept positions in ascending order through two
//     block-wide prefix sums per chunk.
// The result is unique (ties go to the lower index) and bit-exact.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkItems = 8;  // consecutive scores per thread per chunk

// Exclusive prefix sum of x over the block; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int x, int* sm, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kTkWaves ? sm[lane] : 0;
#pragma unroll
    for (int o = 1; o < kTkWaves; o <<= 1) {
      const int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kTkWaves) sm[kTkWaves + lane] = w;
  }
  __syncthreads();
  const int before = wave ? sm[kTkWaves + wave - 1] : 0;
  *total = sm[2 * kTkWaves - 1];
  __syncthreads();
  return before + v - x;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(
    const uint32_t* __restrict__ scores, int H, int n_c, int mode, int seg_len,
    int k, int nseg, int64_t* __restrict__ offsets, int32_t* __restrict__ idx) {
  __shared__ int hist[2048];
  __shared__ int sm[2 * kTkWaves];
  __shared__ int sel[2];

  const int tid = threadIdx.x;
  const int seg = blockIdx.x;
  const uint32_t* data = scores + (size_t)seg * seg_len;
  const int64_t out_base = (int64_t)seg * k;

  // ---- 1. radix select of the k-th largest bit pattern -------------------
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int shift = shifts[p];
    const int nb = 1 << widths[p];
    for (int i = tid; i < 2048; i += kTkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < seg_len; j += kTkThreads) {
      const uint32_t v = data[j];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // thread t owns bins nb-1-2t and nb-2-2t (descending order)
    const int b_hi = nb - 1 - 2 * tid, b_lo = b_hi - 1;
    const int h_hi = b_hi >= 0 ? hist[b_hi] : 0;
    const int h_lo = b_lo >= 0 ? hist[b_lo] : 0;
    int tot;
    const int above = block_excl_scan(h_hi + h_lo, sm, &tot);
    if (b_hi >= 0 && above < remaining && remaining <= above + h_hi) {
      sel[0] = b_hi;
      sel[1] = above;
    }
    if (b_lo >= 0 && above + h_hi < remaining && remaining <= above + h_hi + h_lo) {
      sel[0] = b_lo;
      sel[1] = above + h_hi;
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    remaining -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;  // scores equal to T still to keep

  // ---- 2. ordered compaction ---------------------------------------------
  if (mode == 0 && tid == 0) offsets[seg] = out_base;
  if (seg == 0 && tid == 0) offsets[nseg * (mode == 0 ? 1 : H)] = (int64_t)nseg * k;

  int eq_seen = 0, kept_seen = 0;
#pragma unroll 1
  for (int base = 0; base < seg_len; base += kTkThreads * kTkItems) {
    const int j0 = base + tid * kTkItems;
    uint32_t v[kTkItems];
    int neq = 0;
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const int j = j0 + i;
      v[i] = j < seg_len ? data[j] : 0u;
      neq += (j < seg_len && v[i] == T) ? 1 : 0;
    }
    int eq_tot;
    const int eq_before = eq_seen + block_excl_scan(neq, sm, &eq_tot);
    bool keep[kTkItems];
    int nk = 0, e = 0;
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const int j = j0 + i;
      const bool valid = j < seg_len;
      const bool eq = valid && v[i] == T;
      keep[i] = valid && (v[i] > T || (eq && eq_before + e < need_eq));
      e += eq ? 1 : 0;
      nk += keep[i] ? 1 : 0;
    }
    int k_tot;
    int pos = kept_seen + block_excl_scan(nk, sm, &k_tot);
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const int j = j0 + i;
      if (mode == 1 && j < seg_len && j % n_c == 0)
        offsets[(int64_t)seg * H + j / n_c] = out_base + pos;
      if (keep[i]) {
        if (pos < k) idx[out_base + pos] = mode == 1 ? j % n_c : j;
        ++pos;
      }
    }
    eq_seen += eq_tot;
    kept_seen += k_tot;
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int L, int H, int n_c, int mode,
                       int64_t k_per_segment, int64_t* offsets, int32_t* idx,
                       hipStream_t stream) {
  const int nseg = mode == 0 ? L * H : L;
  const int seg_len = mode == 0 ? n_c : H * n_c;
  hipLaunchKernelGGL(topk_kernel, dim3(nseg), dim3(kTkThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(scores), H, n_c, mode,
                     seg_len, (int)k_per_segment, nseg, offsets, idx);
  return hipGetLastError();
}

}  // namespace kvq
