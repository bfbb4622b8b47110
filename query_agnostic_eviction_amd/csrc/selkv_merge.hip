// Gated merge of evicted tokens into kept rows (SelKV page, "Selective KV
// cache merging", section 1: the soft cosine gate g = max(cos(v_e, v_t), 0)
// decides per evicted token how strongly it is merged into its target).
//
// For kept row t of head (l, h) (position idx[t]) and every routed position
// j in src_idx[src_offsets[t] .. src_offsets[t+1]):
//   g_j = max(<v_j, v_t> / (|v_j| |v_t|), 0)   (0 if a norm is 0 or j is
//                                               outside [0, n_c))
//   x_t' = (x_t + sum_j g_j x_j) / (1 + sum_j g_j)   for x in {k, v}
// accumulated in fp32 in list order (deterministic), rounded to bf16
// (nearest-even).  HBM-bound: every routed and kept row is read once, kept
// rows written once.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ void widen8(u32x4 u, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(u[e] << 16);
    x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ u32x4 narrow8(const float* x) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    u[e] = f32_to_bf16_rne(x[2 * e]) | (f32_to_bf16_rne(x[2 * e + 1]) << 16);
  return u;
}

// Sum over the LPR lanes of a row group (aligned, LPR in {8, 16, 32}).
// Within a 16-lane row the butterfly runs on DPP lane permutations (no LDS
// round trip): swap neighbours, swap pairs, mirror the 8-lane halves (which
// adds the other quad's sum), mirror the row (which adds the other half's);
// the two rows of a 32-lane group are then combined by a lane shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row groups of 8, 16 or 32 lanes");
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);  // row_half_mirror: lane 7 - i within each 8
  if constexpr (LPR >= 16) x += dpp_f32<0x140>(x);  // row_mirror: 15 - i
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

constexpr int kBatch = 1;  // routed rows per step (more costs registers and waves)
constexpr int kMergeLdsHeads = 512;   // offsets staged in LDS up to this many heads

// A row group of D/8 lanes owns one kept row (8 elements, one 16-byte load
// per lane and row); a wave holds 512/D rows.  Routed rows are read kBatch at
// a time (one: with ~68 VGPRs, many waves per SIMD keep enough loads in
// flight, and larger batches measured slower); lanes whose list is exhausted are
// masked off the loads (the wave iterates over its longest list), and the
// workgroup hands its rows to the waves longest list first, so that rows of
// similar length share a wave.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(
    const uint16_t* __restrict__ k_ctx, const uint16_t* __restrict__ v_ctx,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ idx,
    const int64_t* __restrict__ src_offsets, const int32_t* __restrict__ src_idx,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, float* __restrict__ gate,
    float* __restrict__ mass, int LH, int64_t n_c, int64_t total, int64_t n_src) {
  constexpr int LPR = D / 8;     // lanes per row
  constexpr int RPW = 64 / LPR;  // rows per wave
  __shared__ int64_t off_lds[kMergeLdsHeads];
  constexpr int RPB = 4 * RPW;   // rows per workgroup
  __shared__ int cnt_lds[RPB], perm[RPB];
  const int lane = threadIdx.x & 63, sub = lane % LPR;
  // rows of the workgroup ordered by the length of their routed list
  // (longest first, ties by position), so that the rows sharing a wave have
  // similar lengths: a wave runs to the longest list among its rows
  const int64_t t_base = (int64_t)blockIdx.x * RPB;
  if (threadIdx.x < RPB) {
    const int64_t r = t_base + threadIdx.x;
    int c = -1;  // rows past the end sort last
    if (r < total) {
      int64_t a0 = src_offsets[r], a1 = src_offsets[r + 1];
      a0 = a0 < 0 ? 0 : (a0 > n_src ? n_src : a0);
      a1 = a1 < a0 ? a0 : (a1 > n_src ? n_src : a1);
      const int64_t len = a1 - a0;
      c = len > (1 << 30) ? (1 << 30) : (int)len;
    }
    cnt_lds[threadIdx.x] = c;
  }
  __syncthreads();
  if (threadIdx.x < RPB) {
    const int ci = cnt_lds[threadIdx.x];
    int rank = 0;
    for (int j = 0; j < RPB; ++j) {
      const int cj = cnt_lds[j];
      rank += (cj > ci || (cj == ci && j < (int)threadIdx.x)) ? 1 : 0;
    }
    perm[rank] = threadIdx.x;
  }
  __syncthreads();
  const int64_t t = t_base + perm[(threadIdx.x >> 6) * RPW + lane / LPR];
  const bool active = t < total;
  const int64_t tt = active ? t : total - 1;  // inactive groups shadow a valid row
  // head of row tt: the largest lh with offsets[lh] <= tt, searched in LDS
  // when the offsets fit (one coalesced load instead of a chain of
  // dependent global loads)
  const bool staged = LH <= kMergeLdsHeads;
  if (staged) {
    for (int i = threadIdx.x; i < LH; i += 256) off_lds[i] = offsets[i];
    __syncthreads();
  }
  int a = 0, b = LH - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    const int64_t o = staged ? off_lds[mid] : offsets[mid];
    if (o <= tt) a = mid; else b = mid - 1;
  }
  const uint16_t* kh = k_ctx + (int64_t)a * n_c * D + sub * 8;
  const uint16_t* vh = v_ctx + (int64_t)a * n_c * D + sub * 8;
  const int64_t jt = idx[tt];
  const bool row_ok = active && jt >= 0 && jt < n_c;
  const int64_t jt_safe = row_ok ? jt : 0;
  // routed range, clamped to the src_idx array whatever the offsets hold
  int64_t s0 = src_offsets[tt], s1 = src_offsets[tt + 1];
  s0 = s0 < 0 ? 0 : (s0 > n_src ? n_src : s0);
  s1 = s1 < s0 ? s0 : (s1 > n_src ? n_src : s1);
  if (!active) s1 = s0;

  float ks[8], vs[8], vt[8];
  widen8(ldg16_once(kh + jt_safe * D), ks);
  widen8(ldg16_once(vh + jt_safe * D), vt);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (!row_ok) ks[e] = vt[e] = 0.f;
    vs[e] = vt[e];
  }
  float nt2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) nt2 = fmaf(vt[e], vt[e], nt2);
  nt2 = group_sum<LPR>(nt2);
  const float nt = __builtin_sqrtf(nt2);

  // the wave iterates over the longest routed list among its rows
  int64_t steps = s1 - s0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int64_t other = __shfl_xor(steps, o);
    steps = other > steps ? other : steps;
  }
  float msum = 0.f;
  for (int64_t it = 0; it < steps; it += kBatch) {
    u32x4 kr[kBatch], vr[kBatch];
    bool ok[kBatch], in[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t sb = s0 + it + u;
      in[u] = sb < s1;
      const int64_t j = in[u] ? src_idx[sb] : -1;
      ok[u] = row_ok && in[u] && j >= 0 && j < n_c;
      // a lane past the end of its list (or with a rejected position)
      // issues no load: rows of a wave hold lists of different lengths, and
      // the wave runs to the longest of them
      if (ok[u]) {
        kr[u] = ldg16_once(kh + j * D);
        vr[u] = ldg16_once(vh + j * D);
      } else {
        kr[u] = u32x4{0, 0, 0, 0};
        vr[u] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      float kj[8], vj[8];
      widen8(kr[u], kj);
      widen8(vr[u], vj);
      float dot = 0.f, ne2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dot = fmaf(vj[e], vt[e], dot);
        ne2 = fmaf(vj[e], vj[e], ne2);
      }
      dot = group_sum<LPR>(dot);
      ne2 = group_sum<LPR>(ne2);
      float g = 0.f;
      if (ok[u] && ne2 > 0.f && nt2 > 0.f) g = __builtin_fmaxf(dot / (__builtin_sqrtf(ne2) * nt), 0.f);
      if (gate != nullptr && in[u] && sub == 0) gate[s0 + it + u] = g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ks[e] = fmaf(g, kj[e], ks[e]);
        vs[e] = fmaf(g, vj[e], vs[e]);
      }
      msum += g;
    }
  }
  if (!active) return;
  const float w = 1.f + msum;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ks[e] = ks[e] / w;
    vs[e] = vs[e] / w;
  }
  // written once and not read again here: non-temporal stores
  stg16_once(k_out + t * D + sub * 8, narrow8(ks));
  stg16_once(v_out + t * D + sub * 8, narrow8(vs));
  if (mass != nullptr && sub == 0) mass[t] = msum;
}

template <int D>
hipError_t launch_merge_d(const uint16_t* k_ctx, const uint16_t* v_ctx, const int64_t* offsets,
                          const int32_t* idx, const int64_t* src_offsets,
                          const int32_t* src_idx, uint16_t* k_out, uint16_t* v_out,
                          float* gate, float* mass, int LH, int64_t n_c, int64_t total,
                          int64_t n_src, hipStream_t stream) {
  const int64_t rows_per_block = 4 * (512 / D);
  const int64_t blocks = (total + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, k_ctx,
                     v_ctx, offsets, idx, src_offsets, src_idx, k_out, v_out, gate, mass, LH,
                     n_c, total, n_src);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const uint16_t* k_ctx, const uint16_t* v_ctx, const int64_t* offsets,
                        const int32_t* idx, const int64_t* src_offsets, const int32_t* src_idx,
                        uint16_t* k_out, uint16_t* v_out, float* gate, float* mass, int LH,
                        int d, int64_t n_c, int64_t total, int64_t n_src, hipStream_t stream) {
  switch (d) {
    case 64: return launch_merge_d<64>(k_ctx, v_ctx, offsets, idx, src_offsets, src_idx, k_out, v_out, gate, mass, LH, n_c, total, n_src, stream);
    case 128: return launch_merge_d<128>(k_ctx, v_ctx, offsets, idx, src_offsets, src_idx, k_out, v_out, gate, mass, LH, n_c, total, n_src, stream);
    case 256: return launch_merge_d<256>(k_ctx, v_ctx, offsets, idx, src_offsets, src_idx, k_out, v_out, gate, mass, LH, n_c, total, n_src, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
