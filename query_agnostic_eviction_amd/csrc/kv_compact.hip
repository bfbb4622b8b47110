// Compaction of the cache to the kept pairs (KVzip page, "KVzip:
// Query-Agnostic KV Cache Compression with Context Reconstruction", section
// 2.1: the pruned cache KV_p is a subset of KV_c).
//
//   k_out[t] = k_ctx[l][h][idx[t]],  v_out[t] = v_ctx[l][h][idx[t]]
//   for t in [offsets[l*H+h], offsets[l*H+h+1])
//
// A pure HBM-bound gather: each workgroup copies 32 consecutive output rows
// of K and V with 16-byte vector loads and stores (a row of d bf16 values is
// d/8 such chunks, contiguous in memory).  One wave first resolves each
// row's source (head by binary search of the CSR offsets, then its index)
// into an LDS table, so the copy itself is branch-free.  Every address is
// bounded by (l*H+h) < L*H and 0 <= idx < n_c, so a malformed index yields a
// zero row, never a stray read.  `total` may exceed the kept count
// offsets[L*H] (idx and the outputs sized with spare capacity): rows from
// offsets[L*H] on are neither read nor written.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kCpRows = 32;  // output rows per workgroup (the fewest that
                             // still fill one pass of the block at d = 64;
                             // 2-3 % faster cold than 64, 128 is slower)

// SHARED: one kept set idx[0..shared_k) for every head (token-level
// eviction); output row t is head t / shared_k, entry t % shared_k, and the
// offsets are not read.
template <int D, bool SHARED>
__global__ __launch_bounds__(256) void compact_kernel(
    const uint16_t* __restrict__ k_ctx, const uint16_t* __restrict__ v_ctx,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, int LH,
    int64_t n_c, int64_t total, int64_t shared_k) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 256 / CPR;      // rows per pass of the block
  constexpr int IT = kCpRows / RPI;
  static_assert(IT >= 1 && IT * RPI == kCpRows, "whole passes of the block per workgroup");

  __shared__ int64_t src_row[kCpRows];  // lh * n_c + idx, or -1 for a zero row

  const int64_t t0 = (int64_t)blockIdx.x * kCpRows;
  // rows this call writes: the kept rows, within the caller's total
  const int64_t rows = SHARED ? total : min(total, offsets[LH]);
  if (threadIdx.x < kCpRows) {
    const int64_t t = t0 + threadIdx.x;
    int64_t r = -1;
    if (t < rows) {
      int64_t lo, j;
      if (SHARED) {
        lo = t / shared_k;
        j = idx[t - lo * shared_k];
      } else {
        // head of row t: the largest lh with offsets[lh] <= t
        int a = 0, b = LH - 1;
        while (a < b) {
          const int mid = (a + b + 1) >> 1;
          if (offsets[mid] <= t) a = mid; else b = mid - 1;
        }
        lo = a;
        j = idx[t];
      }
      if (j >= 0 && j < n_c) r = lo * n_c + j;
    }
    src_row[threadIdx.x] = r;
  }
  __syncthreads();

  const int c = threadIdx.x % CPR, rr = threadIdx.x / CPR;
  u32x4 kv[IT], vv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    // branch-free: read a valid row (row 0 for a rejected index), then mask
    const int64_t r = src_row[it * RPI + rr];
    const size_t src = (size_t)(r < 0 ? 0 : r) * D + c * 8;
    const uint32_t keep = r < 0 ? 0u : 0xffffffffu;
    kv[it] = ldg16_once(k_ctx + src) & keep;
    vv[it] = ldg16_once(v_ctx + src) & keep;
  }
  // the outputs are not read again by this kernel: non-temporal stores
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t t = t0 + it * RPI + rr;
    if (t < rows) {
      stg16_once(k_out + (size_t)t * D + c * 8, kv[it]);
      stg16_once(v_out + (size_t)t * D + c * 8, vv[it]);
    }
  }
}

template <int D>
hipError_t launch_compact_d(const uint16_t* k_ctx, const uint16_t* v_ctx,
                            const int64_t* offsets, const int32_t* idx,
                            uint16_t* k_out, uint16_t* v_out, int LH,
                            int64_t n_c, int64_t total, int64_t shared_k,
                            hipStream_t stream) {
  const int64_t grid = (total + kCpRows - 1) / kCpRows;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  if (shared_k > 0)
    hipLaunchKernelGGL((compact_kernel<D, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, k_ctx, v_ctx, offsets, idx, k_out, v_out, LH, n_c,
                       total, shared_k);
  else
    hipLaunchKernelGGL((compact_kernel<D, false>), dim3((unsigned)grid), dim3(256), 0,
                       stream, k_ctx, v_ctx, offsets, idx, k_out, v_out, LH, n_c,
                       total, shared_k);
  return hipGetLastError();
}

// Plain device copy of n16 16-byte chunks: the streaming counterpart of the
// gather above (16-byte non-temporal loads and stores), with kCopyInFlight
// loads in flight per thread before their stores and one pass of a grid
// that covers the whole copy (measured on MI355X: non-temporal stores add
// ~10 %, and four loads in flight with a one-pass grid beat eight or
// sixteen with a grid-stride loop).
constexpr int kCopyInFlight = 4;
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kCopyInFlight + threadIdx.x;
  u32x4 v[kCopyInFlight];
#pragma unroll
  for (int u = 0; u < kCopyInFlight; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    v[u] = i < n16 ? ldg16_once(src + i) : zero16();
  }
#pragma unroll
  for (int u = 0; u < kCopyInFlight; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    if (i < n16) stg16_once(dst + i, v[u]);
  }
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t grid = (n16 + 256 * kCopyInFlight - 1) / (256 * kCopyInFlight);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_compact(const uint16_t* k_ctx, const uint16_t* v_ctx,
                          const int64_t* offsets, const int32_t* idx,
                          uint16_t* k_out, uint16_t* v_out, int LH, int d,
                          int64_t n_c, int64_t total, int64_t shared_k,
                          hipStream_t stream) {
  switch (d) {
    case 64: return launch_compact_d<64>(k_ctx, v_ctx, offsets, idx, k_out, v_out, LH, n_c, total, shared_k, stream);
    case 128: return launch_compact_d<128>(k_ctx, v_ctx, offsets, idx, k_out, v_out, LH, n_c, total, shared_k, stream);
    case 256: return launch_compact_d<256>(k_ctx, v_ctx, offsets, idx, k_out, v_out, LH, n_c, total, shared_k, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
