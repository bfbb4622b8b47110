// Pass 1 of the KVzip score (page "KVzip: Query-Agnostic KV Cache Compression
// with Context Reconstruction", section 3.2): the normaliser of every row of
// A = Softmax(Q K^T), written as a natural-log lse, without storing A.
//
// Row (g, i) of KV head (l, h) sees the n_c cached keys and new keys 0..i.
// lse[l][h][g][i] = ln sum_{seen j} exp(scale * <q_{g,i}, k_j>).
//
// Mapping on gfx950:
//  * A workgroup of 4 waves owns 8 query fragments of 32 rows each (a
//    fragment is 32 consecutive positions of one query head g; fragments of a
//    head are numbered b * G + g over 32-position blocks b).  Each wave keeps
//    its two fragments' queries in registers for the whole key sweep.
//  * Keys stream through LDS in tiles of KT rows (double-buffered, one
//    barrier per tile): first the cached keys, then the new keys up to the
//    workgroup's last position.
//  * Logits come from the 32x32x16 bf16 matrix op with the key tile as the
//    A operand and the queries as B, so each lane holds 16 keys of one query:
//    the running max and sum of the online softmax stay lane-local; the two
//    half-waves that share a query merge once at the end.
//  * exp is taken as exp2 with the scale folded into one FMA per logit.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

template <int D>
struct LseCfg {
  static constexpr int KT = (D == 256) ? 32 : 64;  // keys per LDS tile
  static constexpr int NSUB = KT / 32;
  static constexpr int KS = D / 16;                // k-steps of the 32x32x16 op
  static constexpr int ST = D + 8;                 // LDS row stride (bf16), +16 B pad
  static constexpr int CPR = D / 8;                // 16-byte chunks per key row
  static constexpr int LDPT = KT * CPR / 256;      // chunks per thread per tile
};

template <int D>
__global__ __launch_bounds__(256) void lse_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_ctx,
    const uint16_t* __restrict__ k_new, float* __restrict__ lse, int G,
    int n_c, int n_in, int nfrag_head, int wg_per_head, float c2,
    float scale) {
  using C = LseCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][C::KT * C::ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int lh = logical / wg_per_head;
  // latest positions (most keys) first
  const int wgi = wg_per_head - 1 - logical % wg_per_head;

  // fragment bookkeeping (uniform per wave)
  const int F_first = 8 * wgi;
  const int F_last = min(8 * wgi + 7, nfrag_head - 1);
  const int pos_min = 32 * (F_first / G);
  const int new_len = min(n_in, 32 * (F_last / G + 1));

  int fg[2], fpos0[2];
  bool fvalid[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int F = 8 * wgi + 2 * wave + f;
    fvalid[f] = F < nfrag_head;
    fg[f] = fvalid[f] ? F % G : 0;
    fpos0[f] = fvalid[f] ? 32 * (F / G) : 0;
  }

  // queries of both fragments -> registers (B operand layout)
  bf16x8 bq[2][C::KS];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int pos = fpos0[f] + (lane & 31);
    const bool ok = fvalid[f] && pos < n_in;
    const uint16_t* src =
        q + ((size_t)((size_t)lh * G + fg[f]) * n_in + (ok ? pos : 0)) * D +
        8 * (lane >> 5);
    const uint32_t keep = ok ? 0xffffffffu : 0u;  // padding rows read as zeros
#pragma unroll
    for (int s = 0; s < C::KS; ++s) bq[f][s] = as_bf16x8(ldg16(src + 16 * s) & keep);
  }

  const uint16_t* seg_ptr[2] = {k_ctx + (size_t)lh * n_c * D,
                                k_new + (size_t)lh * n_in * D};
  const int T0 = (n_c + C::KT - 1) / C::KT;
  const int T1 = (new_len + C::KT - 1) / C::KT;
  const int T = T0 + T1;

  u32x4 pre[C::LDPT];
  auto load_tile = [&](int t) {
    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const int len = seg == 0 ? n_c : new_len;
#pragma unroll
    for (int it = 0; it < C::LDPT; ++it) {
      const int c = tid + it * 256;
      const int row = c / C::CPR, col = c % C::CPR;
      const int key = key0 + row;
      // branch-free tail: read the last valid row, then zero it
      const int kc = key < len ? key : len - 1;
      const uint32_t keep = key < len ? 0xffffffffu : 0u;
      pre[it] = ldg16(seg_ptr[seg] + (size_t)kc * D + col * 8) & keep;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::LDPT; ++it) {
      const int c = tid + it * 256;
      const int row = c / C::CPR, col = c % C::CPR;
      *reinterpret_cast<u32x4*>(&sk[buf][row * C::ST + col * 8]) = pre[it];
    }
  };

  float m[2] = {kNegBig, kNegBig};
  float sum[2] = {0.f, 0.f};

  auto update = [&](f32x16 acc, int f, bool masked, int seg, int kbase) {
    if (masked) {
      const int qpos = fpos0[f] + (lane & 31);
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = kbase + acc_row(a, lane);
        const bool vis = seg == 0 ? key < n_c : (key <= qpos && key < n_in);
        acc[a] = vis ? acc[a] : -__builtin_inff();
      }
    }
    float t4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      t4[u] = max3f(acc[4 * u], acc[4 * u + 1],
                    __builtin_fmaxf(acc[4 * u + 2], acc[4 * u + 3]));
    const float tmax = max3f(t4[0], t4[1], __builtin_fmaxf(t4[2], t4[3]));
    const float mn = __builtin_fmaxf(m[f], tmax);
    sum[f] *= fast_exp2((m[f] - mn) * c2);
    m[f] = mn;
    const float nmc = -mn * c2;
    float p[16];
#pragma unroll
    for (int a = 0; a < 16; ++a) p[a] = fast_exp2(__builtin_fmaf(acc[a], c2, nmc));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int a = 0; a < w; ++a) p[a] += p[a + w];
    sum[f] += p[0];
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T) load_tile(t + 1);

    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const bool masked = seg == 0 ? (key0 + C::KT > n_c)
                                 : (key0 + C::KT - 1 > pos_min || key0 + C::KT > n_in);
    const uint16_t* sb = &sk[buf][0];
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      f32x16 acc0 = {}, acc1 = {};
      const uint16_t* arow = sb + (sub * 32 + (lane & 31)) * C::ST + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 16 * s);
        acc0 = mfma32(a, bq[0][s], acc0);
        acc1 = mfma32(a, bq[1][s], acc1);
      }
      update(acc0, 0, masked, seg, key0 + sub * 32);
      update(acc1, 1, masked, seg, key0 + sub * 32);
    }

    if (t + 1 < T) store_tile(buf ^ 1);
    __syncthreads();
  }

  // merge the two half-waves that hold the same query, then store
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const float mo = __shfl_xor(m[f], 32);
    const float so = __shfl_xor(sum[f], 32);
    const float M = __builtin_fmaxf(m[f], mo);
    const float S = sum[f] * fast_exp2((m[f] - M) * c2) + so * fast_exp2((mo - M) * c2);
    const float val = __builtin_fmaf(M, scale, __logf(S));
    const int pos = fpos0[f] + (lane & 31);
    if (lane < 32 && fvalid[f] && pos < n_in)
      lse[((size_t)lh * G + fg[f]) * n_in + pos] = val;
  }
}

template <int D>
hipError_t launch_lse_d(const uint16_t* q, const uint16_t* k_ctx,
                        const uint16_t* k_new, float* lse, const ScoreShape& s,
                        hipStream_t stream) {
  const int nb = (s.n_in + 31) / 32;
  const int nfrag = s.G * nb;
  const int wg_per_head = (nfrag + 7) / 8;
  const long long grid = (long long)s.L * s.H * wg_per_head;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c2 = s.scale * kLog2e;
  hipLaunchKernelGGL(lse_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream,
                     q, k_ctx, k_new, lse, s.G, s.n_c, s.n_in, nfrag,
                     wg_per_head, c2, s.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse(const uint16_t* q, const uint16_t* k_ctx,
                      const uint16_t* k_new, float* lse, const ScoreShape& s,
                      hipStream_t stream) {
  switch (s.d) {
    case 64: return launch_lse_d<64>(q, k_ctx, k_new, lse, s, stream);
    case 128: return launch_lse_d<128>(q, k_ctx, k_new, lse, s, stream);
    case 256: return launch_lse_d<256>(q, k_ctx, k_new, lse, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
