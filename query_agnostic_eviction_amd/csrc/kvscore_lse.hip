// Pass 1 of the KVzip score (page "KVzip: Query-Agnostic KV Cache Compression
// with Context Reconstruction", section 3.2): the normaliser of every row of
// A = Softmax(Q K^T), written as a natural-log lse, without storing A.
//
// Row (g, i) of KV head (l, h) sees the n_c cached keys and new keys 0..i.
// lse[l][h][g][i] = ln sum_{seen j} exp(scale * <q_{g,i}, k_j>).
//
// Mapping on gfx950:
//  * A workgroup of 4 waves owns 8 query fragments of 32 rows each (a
//    fragment is 32 consecutive positions of one query head g; fragments of
//    a head are numbered b * G + g over 32-position blocks b).  Each wave
//    keeps its two fragments' queries in registers for the whole key sweep,
//    so every key operand read from LDS feeds two matrix ops.
//  * Keys stream through LDS in 32 KB tiles (16384 / d keys), double-buffered
//    and filled by LDS-DMA straight from HBM while the previous tile is in
//    use: first the cached keys, then the new keys up to the workgroup's last
//    position.  One barrier per tile.
//  * Logits come from the 32x32x16 bf16 matrix op with the key tile as the
//    A operand and the queries as B, so each lane holds 16 keys of one query:
//    the softmax sums stay lane-local; the two half-waves that share a query
//    merge once at the end.
//  * exp is taken as exp2 with the scale folded into one FMA per logit; the
//    running max is updated lazily (see accumulate), so the hot path has no
//    per-logit max, and masked keys enter as a -inf accumulator seed.
//  * Subtile sums enter each lane's running sum with Kahan compensation
//    (per subtile, not per logit), so 128K-key rows stay at fp32 accuracy.
//  * The loop is software-pipelined by one 32-key subtile so the matrix
//    cores and the VALU/transcendental units work at the same time.  At
//    d = 256 the second set of accumulators would not fit beside two
//    fragments' queries at two waves per SIMD, so there each subtile is
//    reduced right after its own matrix ops (the other wave on the SIMD
//    provides the overlap).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

template <int D>
struct LseCfg {
  static constexpr int KT = Tile<D>::ROWS;  // keys per tile
  static constexpr int NSUB = KT / 32;      // 32-key subtiles per tile
  static constexpr int KS = D / 16;         // k-steps of the 32x32x16 op
  // query fragments per wave: two share each key operand read
  static constexpr int NFQ = 2;
  // one-subtile software pipeline (a second set of accumulators); off at
  // d = 256, where it would not fit at two waves per SIMD
  static constexpr bool PIPE = D != 256;
  static constexpr int FPW = 4 * NFQ;      // fragments per workgroup
};

template <int D>
__global__ __launch_bounds__(256, 2) void lse_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_ctx,
    const uint16_t* __restrict__ k_new, float* __restrict__ lse,
    const ScoreShape sh, int nfrag_head, int wg_per_head, float c2) {
  using C = LseCfg<D>;
  const int G = sh.G, n_c = sh.n_c, n_in = sh.n_in;
  const float scale = sh.scale;
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t sk[2 * TL::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int u = logical / wg_per_head;  // work item: (layer, KV head[, chunk])
  // latest positions (most keys) first
  const int wgi = wg_per_head - 1 - logical % wg_per_head;

  constexpr int NFQ = C::NFQ;
  // fragment bookkeeping (uniform per wave)
  const int F_first = C::FPW * wgi;
  const int F_last = min(C::FPW * wgi + C::FPW - 1, nfrag_head - 1);
  const int pos_min = 32 * (F_first / G);
  const int new_len = min(n_in, 32 * (F_last / G + 1));

  int fg[NFQ], fpos0[NFQ];
  bool fvalid[NFQ];
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    const int F = C::FPW * wgi + NFQ * wave + f;
    fvalid[f] = F < nfrag_head;
    fg[f] = fvalid[f] ? F % G : 0;
    fpos0[f] = fvalid[f] ? 32 * (F / G) : 0;
  }

  // queries of the wave's fragments -> registers (B operand layout)
  bf16x8 bq[NFQ][C::KS];
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    const int pos = fpos0[f] + (lane & 31);
    const bool ok = fvalid[f] && pos < n_in;
    const uint16_t* src = q + map_offset(sh.q, u, sh.inner) +
                          ((size_t)fg[f] * n_in + (ok ? pos : 0)) * D + 8 * (lane >> 5);
    const uint32_t keep = ok ? 0xffffffffu : 0u;  // padding rows read as zeros
#pragma unroll
    for (int s = 0; s < C::KS; ++s) bq[f][s] = as_bf16x8(ldg16(src + 16 * s) & keep);
  }

  const uint16_t* seg_ptr[2] = {k_ctx + map_offset(sh.k_ctx, u, sh.inner),
                                k_new + map_offset(sh.k_new, u, sh.inner)};
  const int T0 = (n_c + C::KT - 1) / C::KT;
  const int T1 = (new_len + C::KT - 1) / C::KT;
  const int T = T0 + T1;

  // per-thread constant parts of the tile loads and of the operand reads
  int src_rel[TL::LOADS];
#pragma unroll
  for (int i = 0; i < TL::LOADS; ++i) src_rel[i] = TL::src_rel(i, tid);
  int rd_off[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) rd_off[s] = TL::read_off(lane, s);

  // LDS-DMA of tile t into buffer `buf`; rows past the segment end re-read
  // its last row (finite values; those keys are masked by the -inf seed)
  auto issue_tile = [&](int t, int buf) {
    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const int len = seg == 0 ? n_c : new_len;
    const uint16_t* base = seg_ptr[seg] + (size_t)key0 * D;
    uint16_t* dst = sk + buf * TL::ELEMS + wave * 64 * 8;
    if (key0 + C::KT <= len) {
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i) lds_dma16(base + src_rel[i], dst + i * 256 * 8);
    } else {
      const int last = len - 1 - key0;
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i) {
        const int r = TL::src_row(i, tid);
        const int rel = src_rel[i] - (r > last ? (r - last) * D : 0);
        lds_dma16(base + rel, dst + i * 256 * 8);
      }
    }
  };

  // Online normaliser per lane and fragment: the lane's keys contribute
  // sum * 2^(m * c2) (raw-dot units).  m is a lazily updated running max: a
  // subtile is first summed against the current m and only if that sum
  // exceeds 2^64 (or is not finite: the first real subtile, as m starts at
  // kNegBig) is m raised to the subtile max and the subtile re-summed.  Sums
  // stay far from overflow (< 2^64 per subtile) and terms far below m only
  // underflow where they are negligible, so the result is exact to fp32
  // rounding while the hot path costs one FMA, one exp2 and one add per logit.
  float m[NFQ], nmc[NFQ];
  // running sums with a compensation term (Kahan): long contexts add
  // thousands of subtile sums of similar size, whose rounding errors would
  // otherwise accumulate
  float sum[NFQ], comp[NFQ];
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    m[f] = kNegBig;
    nmc[f] = -kNegBig * c2;
    sum[f] = comp[f] = 0.f;
  }
  constexpr float kRescaleAt = 18446744073709551616.0f;  // 2^64

  auto accumulate = [&](const f32x16* x) {
    // four running partial sums per fragment keep few temporaries live
    float e[NFQ][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int f = 0; f < NFQ; ++f) e[f][a] = fast_exp2(__builtin_fmaf(x[f][a], c2, nmc[f]));
#pragma unroll
    for (int a = 4; a < 16; ++a)
#pragma unroll
      for (int f = 0; f < NFQ; ++f) e[f][a & 3] += fast_exp2(__builtin_fmaf(x[f][a], c2, nmc[f]));
    float ts[NFQ];
    bool big = false;
#pragma unroll
    for (int f = 0; f < NFQ; ++f) {
      ts[f] = (e[f][0] + e[f][1]) + (e[f][2] + e[f][3]);
      big = big || !(ts[f] <= kRescaleAt);
    }
    if (big) {
      // rare path: raise the running max to this subtile's max and re-sum
#pragma unroll
      for (int f = 0; f < NFQ; ++f) {
        if (ts[f] <= kRescaleAt) continue;
        float tm = x[f][0];
#pragma unroll
        for (int a = 1; a < 16; ++a) tm = __builtin_fmaxf(tm, x[f][a]);
        const float mn = __builtin_fmaxf(m[f], tm);
        const float rescale = fast_exp2((m[f] - mn) * c2);
        sum[f] *= rescale;
        comp[f] *= rescale;
        m[f] = mn;
        nmc[f] = -mn * c2;
        float t = 0.f;
#pragma unroll
        for (int a = 0; a < 16; ++a) t += fast_exp2(__builtin_fmaf(x[f][a], c2, nmc[f]));
        ts[f] = t;
      }
    }
#pragma unroll
    for (int f = 0; f < NFQ; ++f) {
      const float y = ts[f] - comp[f];
      const float t = sum[f] + y;
      comp[f] = (t - sum[f]) - y;
      sum[f] = t;
    }
  };

  // Accumulator seed: 0 for keys a row sees, -inf for keys it must not see
  // (cached-key tail past n_c, new keys past the row's position or past n_in).
  auto seed = [&](int f, int seg, int kbase) {
    f32x16 init;
    // last key this lane's row may see within the segment
    const int qpos = fpos0[f] + (lane & 31);
    const int lim = (seg == 0 ? n_c - 1 : min(qpos, n_in - 1)) - kbase - 4 * (lane >> 5);
#pragma unroll
    for (int a = 0; a < 16; ++a)
      init[a] = (8 * (a >> 2) + (a & 3)) <= lim ? 0.f : -__builtin_inff();
    return init;
  };

  // software pipeline: the MFMAs of one 32-key subtile run while the VALU
  // reduces the previous subtile's logits
  f32x16 p[NFQ];
#pragma unroll
  for (int f = 0; f < NFQ; ++f)
#pragma unroll
    for (int a = 0; a < 16; ++a) p[f][a] = -__builtin_inff();

  // one 32-key subtile; unmasked subtiles start the chain from an inline zero
  auto subtile = [&](const uint16_t* sb, bool masked, int seg, int kbase) {
    f32x16 c[NFQ];
#pragma unroll
    for (int f = 0; f < NFQ; ++f) {
      if (masked) {
        c[f] = seed(f, seg, kbase);
      } else {
        const f32x16 z = {};
        c[f] = z;
      }
    }
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sb + rd_off[s]);
#pragma unroll
      for (int f = 0; f < NFQ; ++f) c[f] = mfma32(a, bq[f][s], c[f]);
    }
    if constexpr (C::PIPE) {
      accumulate(p);
#pragma unroll
      for (int f = 0; f < NFQ; ++f) p[f] = c[f];
    } else {
      accumulate(c);
    }
  };

  // tile t sits in buffer BUF: prefetch t+1 into the other buffer, consume
  // t, then wait for the prefetch and publish it with one barrier
  auto step = [&](int t, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (t + 1 < T) issue_tile(t + 1, BUF ^ 1);
    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const bool masked = seg == 0 ? (key0 + C::KT > n_c)
                                 : (key0 + C::KT - 1 > pos_min || key0 + C::KT > n_in);
    const uint16_t* sb = sk + BUF * TL::ELEMS;
    if (masked) {
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub)
        subtile(sb + sub * 32 * D, true, seg, key0 + sub * 32);
    } else {
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub)
        subtile(sb + sub * 32 * D, false, seg, key0 + sub * 32);
    }
    wait_all_mem();
    __syncthreads();
  };

  issue_tile(0, 0);
  wait_all_mem();
  __syncthreads();
  for (int t = 0; t < T; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < T) step(t + 1, std::integral_constant<int, 1>{});
  }
  if constexpr (C::PIPE) accumulate(p);

  // merge the two half-waves that hold the same query, then store
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    const float own = sum[f] - comp[f];
    const float mo = __shfl_xor(m[f], 32);
    const float so = __shfl_xor(own, 32);
    const float M = __builtin_fmaxf(m[f], mo);
    const float S = own * fast_exp2((m[f] - M) * c2) + so * fast_exp2((mo - M) * c2);
    const float val = __builtin_fmaf(M, scale, __logf(S));
    const int pos = fpos0[f] + (lane & 31);
    if (lane < 32 && fvalid[f] && pos < n_in)
      lse[map_offset(sh.lse, u, sh.inner) + (size_t)fg[f] * n_in + pos] = val;
  }
}

template <int D>
hipError_t launch_lse_d(const uint16_t* q, const uint16_t* k_ctx,
                        const uint16_t* k_new, float* lse, const ScoreShape& s,
                        hipStream_t stream) {
  const int nb = (s.n_in + 31) / 32;
  const int nfrag = s.G * nb;
  const int wg_per_head = (nfrag + LseCfg<D>::FPW - 1) / LseCfg<D>::FPW;
  const long long grid = (long long)s.nheads * wg_per_head;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c2 = s.scale * kLog2e;
  hipLaunchKernelGGL(lse_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream,
                     q, k_ctx, k_new, lse, s, nfrag, wg_per_head, c2);
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
