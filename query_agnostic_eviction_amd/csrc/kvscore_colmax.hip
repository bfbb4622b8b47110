// Pass 2 of the KVzip score (page "KVzip: Query-Agnostic KV Cache Compression
// with Context Reconstruction", section 3.2): slice A to the cached-key
// columns and take the max over all G grouped queries and all n_in rows
// (the displayed max equation of that section), without storing A.
//
//   scores[l][h][j] = max_{g,i} exp(scale * <q_{g,i}, k_j> - lse[l][h][g][i])
//
// Every row sees every cached key (only the new keys are causal), so this is
// a dense (G * n_in) x n_c product reduced by column.  Because exp is
// monotone, max_i exp(t_i) = exp(max_i t_i): no per-logit exp is needed.
//
// Mapping on gfx950:
//  * A workgroup of 4 waves owns 256 cached keys (2 fragments of 32 per
//    wave, kept in registers as the B operand); it sweeps all G * n_in query
//    rows of its head, staged through LDS in double-buffered tiles.
//  * The accumulator of each 32x32x16 product is seeded with -lse / scale of
//    its rows, so the matrix op itself yields q.k - lse / scale; each lane
//    holds 16 rows of one key and keeps a lane-local running max.
//  * The loop is software-pipelined: the next subtile's operands are read
//    from LDS and the previous subtile's products reduced while the matrix
//    cores work on the current one.
//  * No atomics: each workgroup owns its columns, writes them once, and the
//    result is independent of scheduling.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D>
struct ColCfg {
  static constexpr int QT = (D == 256) ? 32 : 64;  // query rows per LDS tile
  static constexpr int NSUB = QT / 32;
  static constexpr int KS = D / 16;
  static constexpr int ST = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int LDPT = QT * CPR / 256;
};

template <int D>
__global__ __launch_bounds__(256) void colmax_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_ctx,
    const float* __restrict__ lse, float* __restrict__ scores, int G, int n_c,
    int n_in, int wg_per_head, float c2, float inv_scale) {
  using C = ColCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sq[2][C::QT * C::ST];
  __shared__ __attribute__((aligned(16))) float snl[2][C::QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int lh = logical / wg_per_head;
  const int j0 = (logical % wg_per_head) * 256;

  // this wave's two key fragments -> registers (B operand layout)
  bf16x8 bk[2][C::KS];
  int key[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    key[f] = j0 + 32 * (2 * wave + f) + (lane & 31);
    const bool ok = key[f] < n_c;
    const uint16_t* src =
        k_ctx + ((size_t)lh * n_c + (ok ? key[f] : 0)) * D + 8 * (lane >> 5);
    const uint32_t keep = ok ? 0xffffffffu : 0u;  // keys past n_c read as zeros
#pragma unroll
    for (int s = 0; s < C::KS; ++s) bk[f][s] = as_bf16x8(ldg16(src + 16 * s) & keep);
  }

  const int R = G * n_in;  // flattened (g, i) rows of this head
  const uint16_t* qh = q + (size_t)lh * R * D;
  const float* lh_lse = lse + (size_t)lh * R;
  const int T = (R + C::QT - 1) / C::QT;

  u32x4 pre[C::LDPT];
  float pre_nl = 0.f;
  bool pre_ok = false;
  auto load_tile = [&](int t) {
    const int r0 = t * C::QT;
#pragma unroll
    for (int it = 0; it < C::LDPT; ++it) {
      const int c = tid + it * 256;
      const int row = c / C::CPR, col = c % C::CPR;
      // past the last row re-read it: finite values, and the -inf seed of
      // a padding row keeps it out of the max.  Nothing here touches the
      // loaded data, so the loads stay in flight across the compute.
      const int r = r0 + row;
      pre[it] = ldg16(qh + (size_t)(r < R ? r : R - 1) * D + col * 8);
    }
    if (tid < C::QT) {
      const int r = r0 + tid;
      pre_nl = lh_lse[r < R ? r : R - 1];
      pre_ok = r < R;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::LDPT; ++it) {
      const int c = tid + it * 256;
      const int row = c / C::CPR, col = c % C::CPR;
      *reinterpret_cast<u32x4*>(&sq[buf][row * C::ST + col * 8]) = pre[it];
    }
    if (tid < C::QT) snl[buf][tid] = pre_ok ? -pre_nl * inv_scale : -__builtin_inff();
  };

  float M[2] = {-__builtin_inff(), -__builtin_inff()};

  // operands of one 32-row subtile: the query rows (A) and their seeds
  struct Sub {
    bf16x8 a[C::KS];
    f32x16 init;
  };
  auto read_sub = [&](int buf, int sub, Sub& o) {
    const uint16_t* arow =
        &sq[buf][(sub * 32 + (lane & 31)) * C::ST + 8 * (lane >> 5)];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      o.a[s] = *reinterpret_cast<const bf16x8*>(arow + 16 * s);
    // seed: -lse / scale of the 16 rows this lane holds
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(
          &snl[buf][sub * 32 + 8 * grp + 4 * (lane >> 5)]);
      o.init[4 * grp + 0] = v[0];
      o.init[4 * grp + 1] = v[1];
      o.init[4 * grp + 2] = v[2];
      o.init[4 * grp + 3] = v[3];
    }
  };
  auto reduce2 = [&](const f32x16& x0, const f32x16& x1) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      M[0] = max3f(M[0], x0[4 * u], max3f(x0[4 * u + 1], x0[4 * u + 2], x0[4 * u + 3]));
      M[1] = max3f(M[1], x1[4 * u], max3f(x1[4 * u + 1], x1[4 * u + 2], x1[4 * u + 3]));
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // software pipeline: operands of the next subtile are read from LDS and
  // the previous subtile's results reduced while the matrix cores run
  f32x16 p0, p1;
#pragma unroll
  for (int a = 0; a < 16; ++a) p0[a] = p1[a] = -__builtin_inff();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T) load_tile(t + 1);
    Sub cur;
    read_sub(buf, 0, cur);
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      Sub nxt;
      if (sub + 1 < C::NSUB) read_sub(buf, sub + 1, nxt);
      f32x16 c0 = cur.init, c1 = cur.init;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        c0 = mfma32(cur.a[s], bk[0][s], c0);
        c1 = mfma32(cur.a[s], bk[1][s], c1);
      }
      reduce2(p0, p1);
      p0 = c0;
      p1 = c1;
      if (sub + 1 < C::NSUB) cur = nxt;
    }
    if (t + 1 < T) store_tile(buf ^ 1);
    __syncthreads();
  }
  reduce2(p0, p1);

#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const float mx = __builtin_fmaxf(M[f], __shfl_xor(M[f], 32));
    // the exact score is a probability, so never above 1
    const float sc = __builtin_fminf(fast_exp2(mx * c2), 1.0f);
    if (lane < 32 && key[f] < n_c) scores[(size_t)lh * n_c + key[f]] = sc;
  }
}

template <int D>
hipError_t launch_colmax_d(const uint16_t* q, const uint16_t* k_ctx,
                           const float* lse, float* scores, const ScoreShape& s,
                           hipStream_t stream) {
  const int wg_per_head = (s.n_c + 255) / 256;
  const long long grid = (long long)s.L * s.H * wg_per_head;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c2 = s.scale * kLog2e;
  const float inv_scale = (float)(1.0 / (double)s.scale);
  hipLaunchKernelGGL(colmax_kernel<D>, dim3((unsigned)grid), dim3(256), 0,
                     stream, q, k_ctx, lse, scores, s.G, s.n_c, s.n_in,
                     wg_per_head, c2, inv_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_colmax(const uint16_t* q, const uint16_t* k_ctx,
                         const float* lse, float* scores, const ScoreShape& s,
                         hipStream_t stream) {
  switch (s.d) {
    case 64: return launch_colmax_d<64>(q, k_ctx, lse, scores, s, stream);
    case 128: return launch_colmax_d<128>(q, k_ctx, lse, scores, s, stream);
    case 256: return launch_colmax_d<256>(q, k_ctx, lse, scores, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
