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

// ---------------------------------------------------------------------------
// Model-wide budget (mode 2): one top-k over all L*H*n_c scores, run as a
// grid-wide radix select.  Every step is its own launch on the stream, with
// the state in the caller's workspace:
//   init  -> 3 x (histogram over the whole array, pick the bin)  -> T
//   count (per block: scores > T and == T) -> scan over blocks -> ordered
//   write (kept positions, CSR offsets at head boundaries).
// ---------------------------------------------------------------------------
constexpr int kGThreads = 256;
constexpr int kGItems = 16;                  // scores per thread per chunk
constexpr int kGChunk = kGThreads * kGItems;

struct GlobalState {
  unsigned long long hist[2048];
  unsigned long long remaining;  // scores equal to the prefix still to keep
  unsigned int prefix, pmask;
};

__global__ void gsel_init(GlobalState* st, long long k, int64_t* offsets, int nheads) {
  for (int i = threadIdx.x; i < 2048; i += blockDim.x) st->hist[i] = 0;
  if (threadIdx.x == 0) {
    st->remaining = (unsigned long long)k;
    st->prefix = 0;
    st->pmask = 0;
    offsets[nheads] = k;
  }
}

__global__ __launch_bounds__(kGThreads) void gsel_hist(const uint32_t* __restrict__ data,
                                                       long long n, long long per_block,
                                                       GlobalState* st, int shift, int width) {
  __shared__ unsigned int h[2048];
  for (int i = threadIdx.x; i < 2048; i += kGThreads) h[i] = 0;
  __syncthreads();
  const unsigned int prefix = st->prefix, pmask = st->pmask, nb = 1u << width;
  const long long b0 = (long long)blockIdx.x * per_block;
  const long long b1 = b0 + per_block < n ? b0 + per_block : n;
  for (long long j = b0 + threadIdx.x; j < b1; j += kGThreads) {
    const uint32_t v = data[j];
    if ((v & pmask) == prefix) atomicAdd(&h[(v >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (int)nb; i += kGThreads)
    if (h[i]) atomicAdd(&st->hist[i], (unsigned long long)h[i]);
}

// One block of 1024 threads: the bin that holds the remaining-th largest.
__global__ __launch_bounds__(kTkThreads) void gsel_pick(GlobalState* st, int shift, int width) {
  __shared__ unsigned long long wsum[kTkWaves];
  __shared__ unsigned long long sel[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = 1 << width;
  const unsigned long long rem = st->remaining;
  // thread t owns bins nb-1-2t and nb-2-2t (descending); 64-bit prefix sums
  const int b_hi = nb - 1 - 2 * tid, b_lo = b_hi - 1;
  const unsigned long long h_hi = b_hi >= 0 ? st->hist[b_hi] : 0;
  const unsigned long long h_lo = b_lo >= 0 ? st->hist[b_lo] : 0;
  unsigned long long v = h_hi + h_lo, x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  unsigned long long before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const unsigned long long above = before + x - v;
  if (b_hi >= 0 && above < rem && rem <= above + h_hi) { sel[0] = b_hi; sel[1] = above; }
  if (b_lo >= 0 && above + h_hi < rem && rem <= above + h_hi + h_lo) { sel[0] = b_lo; sel[1] = above + h_hi; }
  __syncthreads();
  if (tid == 0) {
    st->prefix |= (unsigned int)sel[0] << shift;
    st->pmask |= (unsigned int)(nb - 1) << shift;
    st->remaining = rem - sel[1];
  }
  // clear the histogram for the next pass
  for (int i = tid; i < 2048; i += kTkThreads) st->hist[i] = 0;
}

__global__ __launch_bounds__(kGThreads) void gsel_count(const uint32_t* __restrict__ data,
                                                        long long n, long long per_block,
                                                        const GlobalState* st,
                                                        unsigned long long* counts) {
  __shared__ unsigned long long red[2][kGThreads / kWave];
  const uint32_t T = st->prefix;
  const long long b0 = (long long)blockIdx.x * per_block;
  const long long b1 = b0 + per_block < n ? b0 + per_block : n;
  unsigned long long eq = 0, gt = 0;
  for (long long j = b0 + threadIdx.x; j < b1; j += kGThreads) {
    const uint32_t v = data[j];
    eq += v == T;
    gt += v > T;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    eq += __shfl_xor(eq, o);
    gt += __shfl_xor(gt, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = eq; red[1][wave] = gt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long e = 0, g = 0;
    for (int w = 0; w < kGThreads / kWave; ++w) { e += red[0][w]; g += red[1][w]; }
    counts[2 * blockIdx.x] = e;
    counts[2 * blockIdx.x + 1] = g;
  }
}

// Inclusive prefix sum of x over a 1024-thread block (64-bit).
__device__ __forceinline__ unsigned long long block_incl_scan1024(unsigned long long x,
                                                                  unsigned long long* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm[wave] = v;
  __syncthreads();
  unsigned long long before = 0;
  for (int w = 0; w < wave; ++w) before += sm[w];
  __syncthreads();
  return before + v;
}

// One block of 1024 threads, one write-pass block per thread (there are at
// most 1024): turns the per-block counts into the number of equal scores and
// of kept scores before each block.
__global__ __launch_bounds__(kTkThreads) void gsel_scan(const GlobalState* st,
                                                        unsigned long long* counts,
                                                        int nblocks) {
  __shared__ unsigned long long sm[kTkWaves];
  const int b = threadIdx.x;
  const unsigned long long need = st->remaining;
  const unsigned long long e = b < nblocks ? counts[2 * b] : 0;
  const unsigned long long g = b < nblocks ? counts[2 * b + 1] : 0;
  const unsigned long long eq_before = block_incl_scan1024(e, sm) - e;
  const unsigned long long take =
      eq_before >= need ? 0 : (need - eq_before < e ? need - eq_before : e);
  const unsigned long long kept_before = block_incl_scan1024(g + take, sm) - (g + take);
  if (b < nblocks) {
    counts[2 * b] = eq_before;
    counts[2 * b + 1] = kept_before;
  }
}

__device__ __forceinline__ unsigned long long block_excl_scan64(unsigned long long x,
                                                                 unsigned long long* sm,
                                                                 unsigned long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm[wave] = v;
  __syncthreads();
  unsigned long long before = 0, tot = 0;
  for (int w = 0; w < kGThreads / kWave; ++w) {
    if (w < wave) before += sm[w];
    tot += sm[w];
  }
  *total = tot;
  __syncthreads();
  return before + v - x;
}

__global__ __launch_bounds__(kGThreads) void gsel_write(const uint32_t* __restrict__ data,
                                                        long long n, long long per_block,
                                                        int n_c, const GlobalState* st,
                                                        const unsigned long long* counts,
                                                        int64_t* __restrict__ offsets,
                                                        int32_t* __restrict__ idx,
                                                        long long k) {
  __shared__ unsigned long long sm[kGThreads / kWave];
  const uint32_t T = st->prefix;
  const unsigned long long need = st->remaining;
  unsigned long long eq_seen = counts[2 * blockIdx.x];
  unsigned long long kept_seen = counts[2 * blockIdx.x + 1];
  const long long b0 = (long long)blockIdx.x * per_block;
  const long long b1 = b0 + per_block < n ? b0 + per_block : n;
  for (long long base = b0; base < b1; base += kGChunk) {
    const long long j0 = base + (long long)threadIdx.x * kGItems;
    uint32_t v[kGItems];
    unsigned long long neq = 0;
#pragma unroll
    for (int i = 0; i < kGItems; ++i) {
      const long long j = j0 + i;
      v[i] = j < b1 ? data[j] : 0u;
      neq += (j < b1 && v[i] == T) ? 1 : 0;
    }
    unsigned long long eq_tot;
    const unsigned long long eq_before = eq_seen + block_excl_scan64(neq, sm, &eq_tot);
    bool keep[kGItems];
    unsigned long long nk = 0, e = 0;
#pragma unroll
    for (int i = 0; i < kGItems; ++i) {
      const long long j = j0 + i;
      const bool valid = j < b1;
      const bool eq = valid && v[i] == T;
      keep[i] = valid && (v[i] > T || (eq && eq_before + e < need));
      e += eq ? 1 : 0;
      nk += keep[i] ? 1 : 0;
    }
    unsigned long long k_tot;
    unsigned long long pos = kept_seen + block_excl_scan64(nk, sm, &k_tot);
#pragma unroll
    for (int i = 0; i < kGItems; ++i) {
      const long long j = j0 + i;
      if (j < b1 && j % n_c == 0) offsets[j / n_c] = (int64_t)pos;
      if (keep[i]) {
        if ((long long)pos < k) idx[pos] = (int32_t)(j % n_c);
        ++pos;
      }
    }
    eq_seen += eq_tot;
    kept_seen += k_tot;
  }
}

// Head-level static score (KVzip page, section 4.2): the max of a head's
// pair scores along the sequence.  One 256-thread block per (l, h), eight
// independent loads in flight per thread.
__global__ __launch_bounds__(256) void head_max_kernel(const float* __restrict__ scores,
                                                       int n_c, float* __restrict__ out) {
  __shared__ float red[4];
  const float* s = scores + (size_t)blockIdx.x * n_c;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = -__builtin_inff();
  int j = threadIdx.x;
  for (; j + 7 * 256 < n_c; j += 8 * 256) {
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = __builtin_fmaxf(m[u], s[j + u * 256]);
  }
  for (; j < n_c; j += 256) m[0] = __builtin_fmaxf(m[0], s[j]);
  float r = m[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) r = __builtin_fmaxf(r, m[u]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r = __builtin_fmaxf(r, __shfl_xor(r, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0)
    out[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]),
                                      __builtin_fmaxf(red[2], red[3]));
}

}  // namespace

size_t global_select_workspace(long long n) {
  const long long per_block = global_select_per_block(n);
  const long long nblocks = (n + per_block - 1) / per_block;
  return sizeof(GlobalState) + 16 * (size_t)nblocks + 256;
}

long long global_select_per_block(long long n) {
  // about 4 blocks per CU, each a whole number of write-pass chunks
  long long per = (n + 1023) / 1024;
  per = (per + kGChunk - 1) / kGChunk * kGChunk;
  return per < kGChunk ? kGChunk : per;
}

hipError_t launch_global_topk(const float* scores, long long n, int n_c, int nheads,
                              long long k, int64_t* offsets, int32_t* idx,
                              void* workspace, hipStream_t stream) {
  const long long per_block = global_select_per_block(n);
  const long long nblocks_ll = (n + per_block - 1) / per_block;
  if (n < 1 || nblocks_ll > kTkThreads) return hipErrorInvalidValue;  // gsel_scan's limit
  const int nblocks = (int)nblocks_ll;
  GlobalState* st = reinterpret_cast<GlobalState*>(workspace);
  unsigned long long* counts = reinterpret_cast<unsigned long long*>(
      reinterpret_cast<char*>(workspace) + ((sizeof(GlobalState) + 255) / 256) * 256);
  const uint32_t* data = reinterpret_cast<const uint32_t*>(scores);
  hipLaunchKernelGGL(gsel_init, dim3(1), dim3(256), 0, stream, st, k, offsets, nheads);
  const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL(gsel_hist, dim3(nblocks), dim3(kGThreads), 0, stream, data, n,
                       per_block, st, shifts[p], widths[p]);
    hipLaunchKernelGGL(gsel_pick, dim3(1), dim3(kTkThreads), 0, stream, st, shifts[p],
                       widths[p]);
  }
  hipLaunchKernelGGL(gsel_count, dim3(nblocks), dim3(kGThreads), 0, stream, data, n,
                     per_block, st, counts);
  hipLaunchKernelGGL(gsel_scan, dim3(1), dim3(kTkThreads), 0, stream, st, counts, nblocks);
  hipLaunchKernelGGL(gsel_write, dim3(nblocks), dim3(kGThreads), 0, stream, data, n,
                     per_block, n_c, st, counts, offsets, idx, k);
  return hipGetLastError();
}

hipError_t launch_head_max(const float* scores, int nheads, int n_c, float* out,
                           hipStream_t stream) {
  hipLaunchKernelGGL(head_max_kernel, dim3(nheads), dim3(256), 0, stream, scores, n_c, out);
  return hipGetLastError();
}

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
