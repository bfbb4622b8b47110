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
// A segment of up to 32,768 scores (a head of up to 32K cached pairs) is
// first staged in LDS (128 KB), so the four passes read global memory once;
// longer segments are read by each pass.  The result is unique (ties go to
// the lower index) and bit-exact.
#include <mutex>

#include "kvq_device.h"
#include "kvq_internal.h"

// Device memory of kv_topk_select_noalloc: the grid-wide select's state and
// per-block counts (global_select_workspace bytes, at most ~33 KiB for any
// input).  One copy per GPU, held until the process ends.  Host code must
// never pass this name to a kernel or a copy: it is a host-side stand-in;
// the device address comes from noalloc_scratch below.
static __device__ __align__(256) unsigned char scratch[kvq::kNoAllocScratchBytes];

namespace kvq {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkItems = 8;  // consecutive scores per thread per chunk
constexpr int kHistBatch = 16;  // loads in flight per thread in a histogram pass

// The DPP value of lane i's partner under ctrl (0 where the partner is out
// of range, or in rows row_mask leaves out).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP lane
// permutations, with no LDS round trip: a shift-and-add ladder within each
// 16-lane row (row_shr 1, 2, 4, 8), then the last lane of row 0 (and of
// row 2) broadcast into the next row, and the last lane of row 1 into rows
// 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i32<0x111>(v);        // row_shr:1
  v += dpp_i32<0x112>(v);        // row_shr:2
  v += dpp_i32<0x114>(v);        // row_shr:4
  v += dpp_i32<0x118>(v);        // row_shr:8
  v += dpp_i32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_i32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum of x over the block; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int x, int* sm, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v = wave_incl_scan(x);
  if (lane == 63) sm[wave] = v;
  __syncthreads();
  if (wave == 0) {
    const int w = wave_incl_scan(lane < kTkWaves ? sm[lane] : 0);
    if (lane < kTkWaves) sm[kTkWaves + lane] = w;
  }
  __syncthreads();
  const int before = wave ? sm[kTkWaves + wave - 1] : 0;
  *total = sm[2 * kTkWaves - 1];
  __syncthreads();
  return before + v - x;
}

// Order-preserving map of a float's bits to uint32: identity for the
// non-negative scores of the attention path; for signed scores the usual
// sign flip.  In both, -0.0 is folded onto +0.0 so that equal values tie
// (without it a -0.0 score would rank above every positive one).
template <bool SIGNED>
__device__ __forceinline__ uint32_t sort_key(uint32_t v) {
  if (v == 0x80000000u) v = 0u;  // -0.0 ties with +0.0 in both orders
  if (!SIGNED) return v;
  return (v & 0x80000000u) ? ~v : (v | 0x80000000u);
}

// Segments of at most kTkStage scores are staged in LDS once and every pass
// reads them there; longer ones are read from global memory by each pass.
// One 1024-thread block with the full stage fits a compute unit's LDS.
constexpr int kTkStage = 32768;  // 128 KB

template <bool SIGNED, bool STAGED>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(
    const uint32_t* __restrict__ scores, int H, int n_c, int mode, int seg_len,
    int k, int nseg, int64_t* __restrict__ offsets, int32_t* __restrict__ idx) {
  __shared__ int hist[2048];
  __shared__ int sm[2 * kTkWaves];
  __shared__ int sel[2];
  __shared__ uint32_t stage[STAGED ? kTkStage : 1];

  const int tid = threadIdx.x;
  const int seg = blockIdx.x;
  const uint32_t* data = scores + (size_t)seg * seg_len;
  const int64_t out_base = (int64_t)seg * k;
  const unsigned useg = (unsigned)seg_len;  // < 2^31: unsigned index math cannot wrap
  if constexpr (STAGED) {
    // kHistBatch loads in flight per thread, then the LDS writes
    for (unsigned base = 0; base < useg; base += kTkThreads * kHistBatch) {
      uint32_t v[kHistBatch];
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const unsigned j = base + u * kTkThreads + tid;
        v[u] = j < useg ? data[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const unsigned j = base + u * kTkThreads + tid;
        if (j < useg) stage[j] = v[u];
      }
    }
    __syncthreads();
  }
  // the bits of score j (j < useg); the sort key is applied by the caller,
  // after the value arrives, so a batch of global loads stays in flight
  auto raw_at = [&](unsigned j) -> uint32_t {
    if constexpr (STAGED) return stage[j];
    else return data[j];
  };

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
    // kHistBatch independent loads in flight per thread, then the atomics
    for (unsigned base = 0; base < useg; base += kTkThreads * kHistBatch) {
      uint32_t v[kHistBatch];
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const unsigned j = base + u * kTkThreads + tid;
        v[u] = j < useg ? raw_at(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const unsigned j = base + u * kTkThreads + tid;
        const uint32_t key = sort_key<SIGNED>(v[u]);
        if (j < useg && (key & pmask) == prefix)
          atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
      }
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
  if (offsets != nullptr) {
    if (mode == 0 && tid == 0) offsets[seg] = out_base;
    if (seg == 0 && tid == 0) offsets[nseg * (mode == 0 ? 1 : H)] = (int64_t)nseg * k;
  }

  int eq_seen = 0, kept_seen = 0;
#pragma unroll 1
  for (unsigned base = 0; base < useg; base += kTkThreads * kTkItems) {
    const unsigned j0 = base + tid * kTkItems;
    uint32_t v[kTkItems];
    int neq = 0;
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const unsigned j = j0 + i;
      v[i] = j < useg ? sort_key<SIGNED>(raw_at(j)) : 0u;
      neq += (j < useg && v[i] == T) ? 1 : 0;
    }
    int eq_tot;
    const int eq_before = eq_seen + block_excl_scan(neq, sm, &eq_tot);
    bool keep[kTkItems];
    int nk = 0, e = 0;
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const unsigned j = j0 + i;
      const bool valid = j < useg;
      const bool eq = valid && v[i] == T;
      keep[i] = valid && (v[i] > T || (eq && eq_before + e < need_eq));
      e += eq ? 1 : 0;
      nk += keep[i] ? 1 : 0;
    }
    int k_tot;
    int pos = kept_seen + block_excl_scan(nk, sm, &k_tot);
#pragma unroll
    for (int i = 0; i < kTkItems; ++i) {
      const unsigned j = j0 + i;
      if (mode == 1 && j < useg && j % (unsigned)n_c == 0)
        offsets[(int64_t)seg * H + j / (unsigned)n_c] = out_base + pos;
      if (keep[i]) {
        if ((unsigned)pos < (unsigned)k)
          idx[out_base + pos] = (int32_t)(mode == 1 ? j % (unsigned)n_c : j);
        ++pos;
      }
    }
    eq_seen += eq_tot;
    kept_seen += k_tot;
  }
}

// ---------------------------------------------------------------------------
// Grid-wide select: one top-k over a long array spread over many workgroups
// (the model-wide budget, mode 2, and the token budget).  The state lives in
// the caller's workspace; the steps are stream-ordered launches, and within
// a launch the last workgroup to finish (an atomic arrival counter, no
// waiting) does the serial part:
//   init -> 3 x hist (last block: pick the bin, clear the histogram)
//        -> count (last block: scan the per-block counts) -> ordered write.
// ---------------------------------------------------------------------------
constexpr int kGThreads = 256;
constexpr int kGItems = 16;                  // scores per thread per chunk
constexpr int kGChunk = kGThreads * kGItems;
constexpr int kGMaxBlocks = 1024;            // bound of the count scan

struct GlobalState {
  unsigned long long hist[2048];
  unsigned long long remaining;  // scores equal to the prefix still to keep
  unsigned int prefix, pmask;
  unsigned int arrived;          // workgroups done in the current launch
};

__device__ __forceinline__ unsigned long long load_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every thread of the workgroup that arrives last in this launch.
// The barrier completes every wave's writes to this die's L2; one
// device-scope fence (an L2 write-back on a multi-die part) then publishes
// them before the arrival is counted.  The last workgroup reads what the
// others published through device-scope loads.
__device__ __forceinline__ bool last_to_arrive(GlobalState* st) {
  __shared__ int last;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    last = atomicAdd(&st->arrived, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  return last;
}

// One step of the 64-bit DPP ladder: v + (lane partner's v), the partner's
// two halves moved by the same permutation (0 where out of range).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ unsigned long long dpp_add64(unsigned long long v) {
  const unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
  const unsigned plo = (unsigned)dpp_i32<CTRL, ROW_MASK>((int)lo);
  const unsigned phi = (unsigned)dpp_i32<CTRL, ROW_MASK>((int)hi);
  return v + (((unsigned long long)phi << 32) | plo);
}

// Exclusive prefix sum over a 256-thread block (64-bit); *total = block sum.
__device__ __forceinline__ unsigned long long block_excl_scan64(unsigned long long x,
                                                                 unsigned long long* sm,
                                                                 unsigned long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the ladder of wave_incl_scan
  unsigned long long v = x;
  v = dpp_add64<0x111>(v);
  v = dpp_add64<0x112>(v);
  v = dpp_add64<0x114>(v);
  v = dpp_add64<0x118>(v);
  v = dpp_add64<0x142, 0xA>(v);
  v = dpp_add64<0x143, 0xC>(v);
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

__global__ void gsel_init(GlobalState* st, long long k, int64_t* offsets, int nheads) {
  for (int i = threadIdx.x; i < 2048; i += blockDim.x) st->hist[i] = 0;
  if (threadIdx.x == 0) {
    st->remaining = (unsigned long long)k;
    st->prefix = 0;
    st->pmask = 0;
    st->arrived = 0;
    if (offsets) offsets[nheads] = k;
  }
}

template <bool SIGNED>
__global__ __launch_bounds__(kGThreads) void gsel_hist(const uint32_t* __restrict__ data,
                                                       long long n, long long per_block,
                                                       GlobalState* st, int shift, int width) {
  __shared__ unsigned int h[2048];
  __shared__ unsigned long long sm[kGThreads / kWave];
  __shared__ unsigned long long sel[2];
  for (int i = threadIdx.x; i < 2048; i += kGThreads) h[i] = 0;
  __syncthreads();
  const unsigned int prefix = st->prefix, pmask = st->pmask, nb = 1u << width;
  const long long b0 = (long long)blockIdx.x * per_block;
  const long long b1 = b0 + per_block < n ? b0 + per_block : n;
  for (long long base = b0; base < b1; base += kGChunk) {
    uint32_t v[kGItems];
#pragma unroll
    for (int u = 0; u < kGItems; ++u) {
      const long long j = base + u * kGThreads + threadIdx.x;
      v[u] = j < b1 ? data[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kGItems; ++u) {
      const long long j = base + u * kGThreads + threadIdx.x;
      const uint32_t key = sort_key<SIGNED>(v[u]);
      if (j < b1 && (key & pmask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (int)nb; i += kGThreads)
    if (h[i]) atomicAdd(&st->hist[i], (unsigned long long)h[i]);
  if (!last_to_arrive(st)) return;

  // last workgroup: the bin holding the remaining-th largest key; thread t
  // owns the 8 bins nb-1-8t .. nb-8-8t (descending)
  const unsigned long long rem = st->remaining;
  unsigned long long c[8], tot8 = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int b = (int)nb - 1 - 8 * (int)threadIdx.x - u;
    c[u] = b >= 0 ? load_agent(&st->hist[b]) : 0ull;
    tot8 += c[u];
  }
  unsigned long long all;
  unsigned long long above = block_excl_scan64(tot8, sm, &all);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int b = (int)nb - 1 - 8 * (int)threadIdx.x - u;
    if (b >= 0 && above < rem && rem <= above + c[u]) { sel[0] = (unsigned)b; sel[1] = above; }
    above += c[u];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2048; i += kGThreads) st->hist[i] = 0;
  if (threadIdx.x == 0) {
    st->prefix = prefix | ((unsigned int)sel[0] << shift);
    st->pmask = pmask | ((nb - 1) << shift);
    st->remaining = rem - sel[1];
    st->arrived = 0;
  }
}

// Per block: scores equal to / above the selected key; the last block turns
// them into the equal and kept counts before each block.
template <bool SIGNED>
__global__ __launch_bounds__(kGThreads) void gsel_count(const uint32_t* __restrict__ data,
                                                        long long n, long long per_block,
                                                        GlobalState* st,
                                                        unsigned long long* counts) {
  __shared__ unsigned long long red[2][kGThreads / kWave];
  __shared__ unsigned long long sm[kGThreads / kWave];
  const uint32_t T = st->prefix;
  const long long b0 = (long long)blockIdx.x * per_block;
  const long long b1 = b0 + per_block < n ? b0 + per_block : n;
  unsigned long long eq = 0, gt = 0;
  for (long long base = b0; base < b1; base += kGChunk) {
    uint32_t v[kGItems];
#pragma unroll
    for (int u = 0; u < kGItems; ++u) {
      const long long j = base + u * kGThreads + threadIdx.x;
      v[u] = j < b1 ? data[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kGItems; ++u) {
      const long long j = base + u * kGThreads + threadIdx.x;
      const uint32_t key = sort_key<SIGNED>(v[u]);
      eq += (j < b1 && key == T) ? 1 : 0;
      gt += (j < b1 && key > T) ? 1 : 0;
    }
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
  if (!last_to_arrive(st)) return;

  // last workgroup: thread t owns blocks 4t .. 4t+3 (gridDim.x <= 1024)
  const int nblocks = (int)gridDim.x;
  const unsigned long long need = st->remaining;
  unsigned long long e[4], g[4], e_sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = 4 * (int)threadIdx.x + u;
    e[u] = b < nblocks ? load_agent(&counts[2 * b]) : 0ull;
    g[u] = b < nblocks ? load_agent(&counts[2 * b + 1]) : 0ull;
    e_sum += e[u];
  }
  unsigned long long tot;
  unsigned long long eq_before = block_excl_scan64(e_sum, sm, &tot);
  unsigned long long kept[4], k_sum = 0, eqb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    eqb[u] = eq_before;
    const unsigned long long take =
        eq_before >= need ? 0 : (need - eq_before < e[u] ? need - eq_before : e[u]);
    kept[u] = g[u] + take;
    k_sum += kept[u];
    eq_before += e[u];
  }
  unsigned long long kept_before = block_excl_scan64(k_sum, sm, &tot);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = 4 * (int)threadIdx.x + u;
    if (b < nblocks) {
      counts[2 * b] = eqb[u];
      counts[2 * b + 1] = kept_before;
    }
    kept_before += kept[u];
  }
  if (threadIdx.x == 0) st->arrived = 0;
}

template <bool SIGNED>
__global__ __launch_bounds__(kGThreads) void gsel_write(const uint32_t* __restrict__ data,
                                                        long long n, long long per_block,
                                                        long long n_c, const GlobalState* st,
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
      v[i] = j < b1 ? sort_key<SIGNED>(data[j]) : 0u;
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
      if (offsets && j < b1 && j % n_c == 0) offsets[j / n_c] = (int64_t)pos;
      if (keep[i]) {
        if (pos < (unsigned long long)k) idx[pos] = (int32_t)(j % n_c);
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

long long global_select_per_block(long long n) {
  // a whole number of chunks per block, at most kGMaxBlocks blocks
  long long per = (n + kGMaxBlocks - 1) / kGMaxBlocks;
  per = (per + kGChunk - 1) / kGChunk * kGChunk;
  return per < kGChunk ? kGChunk : per;
}

size_t global_select_workspace(long long n) {
  const long long per_block = global_select_per_block(n);
  const long long nblocks = (n + per_block - 1) / per_block;
  return ((sizeof(GlobalState) + 255) / 256) * 256 + 16 * (size_t)nblocks;
}

template <bool SIGNED>
static hipError_t launch_global_select(const float* scores, long long n, long long n_c,
                                       int nheads, long long k, int64_t* offsets,
                                       int32_t* idx, void* workspace, hipStream_t stream) {
  const long long per_block = global_select_per_block(n);
  const long long nblocks_ll = (n + per_block - 1) / per_block;
  if (n < 1 || nblocks_ll > kGMaxBlocks) return hipErrorInvalidValue;
  const int nblocks = (int)nblocks_ll;
  GlobalState* st = reinterpret_cast<GlobalState*>(workspace);
  unsigned long long* counts = reinterpret_cast<unsigned long long*>(
      reinterpret_cast<char*>(workspace) + ((sizeof(GlobalState) + 255) / 256) * 256);
  const uint32_t* data = reinterpret_cast<const uint32_t*>(scores);
  hipLaunchKernelGGL(gsel_init, dim3(1), dim3(256), 0, stream, st, k, offsets, nheads);
  const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
  for (int p = 0; p < 3; ++p)
    hipLaunchKernelGGL(gsel_hist<SIGNED>, dim3(nblocks), dim3(kGThreads), 0, stream, data,
                       n, per_block, st, shifts[p], widths[p]);
  hipLaunchKernelGGL(gsel_count<SIGNED>, dim3(nblocks), dim3(kGThreads), 0, stream, data, n,
                     per_block, st, counts);
  hipLaunchKernelGGL(gsel_write<SIGNED>, dim3(nblocks), dim3(kGThreads), 0, stream, data, n,
                     per_block, n_c, st, counts, offsets, idx, k);
  return hipGetLastError();
}

hipError_t launch_global_topk(const float* scores, long long n, int n_c, int nheads,
                              long long k, int64_t* offsets, int32_t* idx,
                              void* workspace, hipStream_t stream) {
  return launch_global_select<false>(scores, n, n_c, nheads, k, offsets, idx, workspace,
                                     stream);
}

hipError_t launch_select_tokens_grid(const float* scores, long long n, long long k,
                                     int32_t* idx, void* workspace, hipStream_t stream) {
  return launch_global_select<true>(scores, n, n, 1, k, nullptr, idx, workspace, stream);
}

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the address of this GPU's copy of the array (the current device's)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
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
  if (seg_len <= kTkStage)
    hipLaunchKernelGGL((topk_kernel<false, true>), dim3(nseg), dim3(kTkThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(scores), H, n_c, mode,
                       seg_len, (int)k_per_segment, nseg, offsets, idx);
  else
    hipLaunchKernelGGL((topk_kernel<false, false>), dim3(nseg), dim3(kTkThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(scores), H, n_c, mode,
                       seg_len, (int)k_per_segment, nseg, offsets, idx);
  return hipGetLastError();
}


}  // namespace kvq
