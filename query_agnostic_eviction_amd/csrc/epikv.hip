// Attention-free token score of the EpiKV page ("EpiKV", section 3.2,
// hidden-state variation signal).
//
// epi_deltas (equation 1): g_l(t) = || h_l(t) - h_l(t-1) ||_2 for t >= 1 and
// g_l(0) = 0 (position 0 has no predecessor).  HBM-bound: every hidden state
// row is read once (plus one row per run of kRun rows).  Squared differences
// are summed in fp32: at most 8 * CH = 32 terms per thread, a 6-level
// butterfly per wave, then the four waves' parts.
//
// epi_scores (equations 2 and 3): per position t >= 1, over the causal
// window of the defined positions max(1, t - w + 1) .. t (the current one
// included), either the window mean (equation 2) or the z-score
// (g(t) - mean) / (population deviation + eps) (equation 3), computed in
// fp64 with a two-pass mean and deviation; the score is band A's mean
// statistic minus band B's.  Position 0 scores 0.  Tiny work: a block stages
// each layer's window span of g through LDS.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kRun = 16;    // consecutive rows per workgroup
constexpr int kGroup = 4;   // rows loaded together (loads in flight per thread)

__device__ __forceinline__ float sq_diff_sum(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a_lo = __uint_as_float(a[e] << 16), a_hi = __uint_as_float(a[e] & 0xffff0000u);
    const float b_lo = __uint_as_float(b[e] << 16), b_hi = __uint_as_float(b[e] & 0xffff0000u);
    const float d0 = a_lo - b_lo, d1 = a_hi - b_hi;
    acc = fmaf(d0, d0, acc);
    acc = fmaf(d1, d1, acc);
  }
  return acc;
}

// One workgroup (4 waves) per run of kRun rows of one layer; thread t owns
// the 16-byte chunks t, t + 256, ... of every row (CH of them, D <= 2048 *
// CH), so each wave streams a contiguous 1 KB slice per chunk.  Each wave
// reduces its part of a row with a butterfly and parks it in LDS; the four
// parts of every row are summed once at the end of the run.
template <int CH>
__global__ __launch_bounds__(256) void epi_deltas_kernel(const uint16_t* __restrict__ h,
                                                         int64_t n, int D,
                                                         int runs_per_layer,
                                                         float* __restrict__ g) {
  __shared__ float part[kRun][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int layer = (int)(blockIdx.x / (unsigned)runs_per_layer);
  const int64_t r0 = (int64_t)(blockIdx.x - (unsigned)layer * runs_per_layer) * kRun;
  const int64_t r1 = r0 + kRun < n ? r0 + kRun : n;
  const int cpr = D >> 3;
  const uint16_t* base = h + (size_t)layer * n * D;

  auto load_row = [&](int64_t r, u32x4* dst) {
    const uint16_t* row = base + (size_t)r * D;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i;
      dst[i] = c < cpr ? ldg16_once(row + c * 8) : u32x4{0, 0, 0, 0};
    }
  };

  u32x4 prev[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) prev[i] = u32x4{0, 0, 0, 0};
  if (r0 > 0) load_row(r0 - 1, prev);
  for (int64_t g0 = r0; g0 < r1; g0 += kGroup) {
    u32x4 rows[kGroup][CH];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) load_row(g0 + u < r1 ? g0 + u : r1 - 1, rows[u]);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < CH; ++i) acc = sq_diff_sum(rows[u][i], u ? rows[u - 1][i] : prev[i], acc);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0 && g0 + u < r1) part[g0 + u - r0][wave] = acc;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) prev[i] = rows[kGroup - 1][i];
  }
  __syncthreads();
  if (tid < r1 - r0) {
    const int64_t r = r0 + tid;
    const float ss = ((part[tid][0] + part[tid][1]) + part[tid][2]) + part[tid][3];
    g[(size_t)layer * n + r] = r == 0 ? 0.f : __builtin_sqrtf(ss);
  }
}

constexpr int kScoreBlock = 256;

__global__ __launch_bounds__(kScoreBlock) void epi_scores_kernel(
    const float* __restrict__ g, int n_a, int n_b, int64_t n, int w, double eps,
    int detrend, float* __restrict__ scores) {
  extern __shared__ float span[];  // w - 1 + kScoreBlock values
  const int64_t t0 = (int64_t)blockIdx.x * kScoreBlock;
  const int64_t t = t0 + threadIdx.x;
  const int64_t s0 = t0 - (w - 1);  // first staged position (may be < 0)
  const int span_len = w - 1 + kScoreBlock;
  double band[2] = {0.0, 0.0};
  for (int l = 0; l < n_a + n_b; ++l) {
    const float* gl = g + (size_t)l * n;
    __syncthreads();
    for (int i = threadIdx.x; i < span_len; i += kScoreBlock) {
      const int64_t p = s0 + i;
      span[i] = (p >= 0 && p < n) ? gl[p] : 0.f;
    }
    __syncthreads();
    if (t >= 1 && t < n) {
      const int64_t lo = t - w + 1 > 1 ? t - w + 1 : 1;
      const int m = (int)(t - lo + 1);
      const float* x = span + (lo - s0);
      double sum = 0.0;
      for (int i = 0; i < m; ++i) sum += (double)x[i];
      const double mean = sum / m;
      double stat = mean;
      if (detrend) {
        double ss = 0.0;
        for (int i = 0; i < m; ++i) {
          const double dv = (double)x[i] - mean;
          ss = fma(dv, dv, ss);
        }
        const double sigma = sqrt(ss / m);
        stat = ((double)x[m - 1] - mean) / (sigma + eps);
      }
      band[l < n_a ? 0 : 1] += stat;
    }
  }
  if (t < n) scores[t] = t == 0 ? 0.f : (float)(band[0] / n_a - band[1] / n_b);
}

template <int CH>
hipError_t launch_deltas_n(const uint16_t* h, int n_layers, int64_t n, int D, float* g,
                           hipStream_t stream) {
  const int64_t runs = (n + kRun - 1) / kRun;
  const int64_t blocks = runs * n_layers;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(epi_deltas_kernel<CH>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     h, n, D, (int)runs, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_epi_deltas(const uint16_t* h, int n_layers, int64_t n, int D, float* g,
                             hipStream_t stream) {
  const int ch = (D / 8 + 255) / 256;
  if (ch <= 1) return launch_deltas_n<1>(h, n_layers, n, D, g, stream);
  if (ch <= 2) return launch_deltas_n<2>(h, n_layers, n, D, g, stream);
  if (ch <= 4) return launch_deltas_n<4>(h, n_layers, n, D, g, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_epi_scores(const float* g, int n_a, int n_b, int64_t n, int w, double eps,
                             int detrend, float* scores, hipStream_t stream) {
  const int64_t blocks = (n + kScoreBlock - 1) / kScoreBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * (size_t)(w - 1 + kScoreBlock);
  hipLaunchKernelGGL(epi_scores_kernel, dim3((unsigned)blocks), dim3(kScoreBlock), lds,
                     stream, g, n_a, n_b, n, w, eps, detrend, scores);
  return hipGetLastError();
}

}  // namespace kvq
