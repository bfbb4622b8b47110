// Pass 1 of the KVzip score (page "KVzip: Query-Agnostic KV Cache Compression
// with Context Reconstruction", section 3.2): the normaliser of every row of
// A = Softmax(Q K^T), written as a natural-log lse, without storing A.
//
// Row (g, i) of KV head (l, h) sees the n_c cached keys and new keys 0..i.
// lse[l][h][g][i] = ln sum_{seen j} exp(scale * <q_{g,i}, k_j>).
//
// Mapping on gfx950:
//  * A workgroup of 4 waves owns 4 * NFQ query fragments of 32 rows each (a
//    fragment is 32 consecutive positions of one query head g; fragments of
//    a head are numbered b * G + g over 32-position blocks b).  Each wave
//    keeps its NFQ fragments' queries in registers for the whole key sweep.
//  * Keys stream through LDS in 32 KB tiles (16384 / d keys), double-buffered
//    and filled by LDS-DMA straight from HBM while the previous tile is in
//    use: first the cached keys, then the new keys up to the workgroup's last
//    position.  One barrier per tile.
//  * Logits come from the 32x32x16 bf16 matrix op with the key tile as the
//    A operand and the queries as B, so each lane holds 16 keys of one query:
//    the softmax sums stay lane-local; the two half-waves that share a query
//    merge once at the end.
//  * A 32-key subtile's key operands are read from LDS once into registers
//    and feed the products of all the wave's fragments (four at d <= 128,
//    two at d = 256, where a fragment's queries take twice the registers),
//    which are staggered: while the matrix core runs the chain of fragment
//    f, the VALU reduces the logits of fragment f - 1 (for f = 0, the last
//    fragment of the previous subtile).  Only two sets of accumulators are
//    live, which is what leaves room for the fragments' queries (128
//    registers).
//  * exp is taken as exp2 with the scale folded into one FMA per logit; the
//    running max is updated lazily (see reduce_t), so the hot path has no
//    per-logit max.  Logits of keys a row must not see are set to -inf after
//    the products of the few subtiles that hold such keys (under a uniform
//    branch).
//  * Sums enter each lane's running sum with Kahan compensation once per
//    tile (a tile's subtile sums are first added plainly), so 128K-key rows
//    stay at fp32 accuracy.
//  * A wave stops computing after the last tile holding a key its rows see
//    (and a wave holding no rows computes nothing); it keeps issuing its
//    share of the tile loads and joining the barriers.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int D>
struct LseCfg {
  static constexpr int KT = Tile<D>::ROWS;  // keys per tile
  static constexpr int NSUB = KT / 32;      // 32-key subtiles per tile
  static constexpr int KS = D / 16;         // k-steps of the 32x32x16 op
  // query fragments per wave: each key operand read feeds NFQ matrix ops
  static constexpr int NFQ = D == 256 ? 2 : 4;
  static constexpr int FPW = 4 * NFQ;      // fragments per workgroup
};

template <int D>
__global__ __launch_bounds__(256, 2) void lse_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_ctx,
    const uint16_t* __restrict__ k_new, float* __restrict__ lse,
    const ScoreShape sh, int nfrag_head, int wg_per_head, float c2) {
  using C = LseCfg<D>;
  using TL = Tile<D>;
  constexpr int NFQ = C::NFQ;
  const int G = sh.G, n_c = sh.n_c, n_in = sh.n_in;
  __shared__ __attribute__((aligned(1024))) uint16_t sk[2 * TL::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int u = logical / wg_per_head;  // work item: (layer, KV head[, chunk])
  // latest positions (most keys) first
  const int wgi = wg_per_head - 1 - logical % wg_per_head;

  // workgroup bookkeeping: its first position and how far its new keys go.
  // (Integer division runs on the vector unit; readfirstlane returns these
  // uniform values to scalar registers, so the per-tile tests that use them
  // stay scalar.)
  const int F_first = C::FPW * wgi;
  const int F_last = min(C::FPW * wgi + C::FPW - 1, nfrag_head - 1);
  const int pos_min = __builtin_amdgcn_readfirstlane(32 * (F_first / G));
  const int new_len = __builtin_amdgcn_readfirstlane(min(n_in, 32 * (F_last / G + 1)));

  // the wave's fragments (uniform per wave)
  int fg[NFQ], fpos0[NFQ];
  bool fvalid[NFQ];
  int wave_last = -1;  // last position a row of this wave holds (-1: none)
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    const int F = C::FPW * wgi + NFQ * wave + f;
    fvalid[f] = F < nfrag_head;
    fg[f] = __builtin_amdgcn_readfirstlane(fvalid[f] ? F % G : 0);
    fpos0[f] = __builtin_amdgcn_readfirstlane(fvalid[f] ? 32 * (F / G) : 0);
    if (fvalid[f]) wave_last = max(wave_last, min(fpos0[f] + 31, n_in - 1));
  }

  // queries of the wave's fragments -> registers (B operand layout); one
  // array per fragment.  (Every helper below is forced inline: a helper left
  // out of line would keep these arrays in scratch memory.)
  bf16x8 bq0[C::KS], bq1[C::KS], bq2[C::KS], bq3[C::KS];
  auto load_q = [&](bf16x8 (&dst)[C::KS], int f) __attribute__((always_inline)) {
    const int pos = fpos0[f] + (lane & 31);
    const bool ok = fvalid[f] && pos < n_in;
    const uint16_t* src = q + map_offset(sh.q, u, sh.inner) +
                          ((size_t)fg[f] * n_in + (ok ? pos : 0)) * D + 8 * (lane >> 5);
    const uint32_t keep = ok ? 0xffffffffu : 0u;  // padding rows read as zeros
#pragma unroll
    for (int s = 0; s < C::KS; ++s) dst[s] = as_bf16x8(ldg16(src + 16 * s) & keep);
  };
  load_q(bq0, 0);
  if constexpr (NFQ > 1) load_q(bq1, 1);
  if constexpr (NFQ > 2) load_q(bq2, 2);
  if constexpr (NFQ > 3) load_q(bq3, 3);
  auto qop = [&](auto f_tag, int s) __attribute__((always_inline)) -> const bf16x8& {
    constexpr int f = decltype(f_tag)::value;
    if constexpr (f == 0) return bq0[s];
    else if constexpr (f == 1) return bq1[s];
    else if constexpr (f == 2) return bq2[s];
    else return bq3[s];
  };

  const uint16_t* seg_ptr[2] = {k_ctx + map_offset(sh.k_ctx, u, sh.inner),
                                k_new + map_offset(sh.k_new, u, sh.inner)};
  const int T0 = (n_c + C::KT - 1) / C::KT;
  const int T1 = (new_len + C::KT - 1) / C::KT;
  const int T = T0 + T1;
  // tiles this wave computes on: every cached-key tile and the new-key
  // tiles up to its last position
  const int Tw = wave_last < 0 ? 0 : T0 + (wave_last + C::KT) / C::KT;

  // Per-thread parts of the tile-load and key-operand addresses (no
  // registers to spare: two values each, combined on the fly)
  const int rel01[2] = {TL::src_rel(0, tid), TL::src_rel(1, tid)};
  const int rd_base = TL::read_base(lane), rd_x = TL::read_x(lane);
  auto load_rel = [&](int i) __attribute__((always_inline)) {
    return TL::src_rel_from(rel01, i);
  };
  auto key_op = [&](const uint16_t* sb, int s) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(sb + rd_base + 16 * (s ^ rd_x));
  };

  // LDS-DMA of tile t into buffer `buf`; rows past the segment end re-read
  // its last row (finite values; those keys are masked)
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const int len = seg == 0 ? n_c : new_len;
    const uint16_t* base = seg_ptr[seg] + (size_t)key0 * D;
    uint16_t* dst = sk + buf * TL::ELEMS + wave * 64 * 8;
    if (key0 + C::KT <= len) {
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i)
        lds_dma16(base + load_rel(i), dst + i * 256 * 8);
    } else {
      const int last = len - 1 - key0;
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i) {
        const int r = TL::src_row(i, tid);
        const int rel = load_rel(i) - (r > last ? (r - last) * D : 0);
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
  // m is kept as nm = -m * c2, the exp2 argument's offset, so the hot path
  // does not form it (rounding is monotone, so raising m is a min on nm and
  // gives the same nm as forming it from the raised m).
  float nm[NFQ];
  // running sums with a compensation term (Kahan): long contexts add
  // thousands of subtile sums of similar size, whose rounding errors would
  // otherwise accumulate
  float sum[NFQ], comp[NFQ];
  // staggered schedule: a tile's subtile sums are added plainly into tp and
  // enter the compensated sum once per tile
  float tp[NFQ];
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    nm[f] = -kNegBig * c2;
    sum[f] = comp[f] = tp[f] = 0.f;
  }
  constexpr float kRescaleAt = 18446744073709551616.0f;  // 2^64

  auto kahan_add = [&](float v, int f) __attribute__((always_inline)) {
    const float y = v - comp[f];
    const float t = sum[f] + y;
    comp[f] = (t - sum[f]) - y;
    sum[f] = t;
  };
  // fold one fragment's 16 logits per lane (a subtile) into its tile sum and,
  // with FOLD, the tile sum into the running sum
  auto reduce_t = [&](const f32x16& x, auto f_tag, auto fold_tag) __attribute__((always_inline)) {
    constexpr int f = decltype(f_tag)::value;
    constexpr bool FOLD = decltype(fold_tag)::value;
    float nmc = nm[f];
    float e[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) e[a] = fast_exp2(__builtin_fmaf(x[a], c2, nmc));
#pragma unroll
    for (int a = 4; a < 16; ++a) e[a & 3] += fast_exp2(__builtin_fmaf(x[a], c2, nmc));
    float ts = (e[0] + e[1]) + (e[2] + e[3]);
    // the whole wave takes the rare path when one lane needs it (for the
    // others it keeps or raises their max and re-sums: the same result up to
    // rounding); a wave-uniform branch keeps the tile loop free of
    // execution-mask handling
    if (__builtin_amdgcn_ballot_w64(!(ts <= kRescaleAt))) {
      float tm = x[0];
#pragma unroll
      for (int a = 1; a < 16; ++a) tm = __builtin_fmaxf(tm, x[a]);
      const float nmn = __builtin_fminf(nm[f], -tm * c2);
      const float rescale = fast_exp2(nmn - nm[f]);
      sum[f] *= rescale;
      comp[f] *= rescale;
      tp[f] *= rescale;
      nm[f] = nmn;
      nmc = nmn;
      float t = 0.f;
#pragma unroll
      for (int a = 0; a < 16; ++a) t += fast_exp2(__builtin_fmaf(x[a], c2, nmc));
      ts = t;
    }
    if constexpr (FOLD) {
      kahan_add(tp[f] + ts, f);
      tp[f] = 0.f;
    } else {
      tp[f] += ts;
    }
  };

  // Masking: logits of keys a row must not see (cached-key tail past n_c, new
  // keys past the row's position or past n_in) become -inf, which the
  // reduction turns into 0.
  auto mask = [&](f32x16& x, int f, int seg, int kbase) __attribute__((always_inline)) {
    // last key this lane's row may see within the segment
    const int qpos = fpos0[f] + (lane & 31);
    const int lim = (seg == 0 ? n_c - 1 : min(qpos, n_in - 1)) - kbase - 4 * (lane >> 5);
#pragma unroll
    for (int a = 0; a < 16; ++a)
      if ((8 * (a >> 2) + (a & 3)) > lim) x[a] = -__builtin_inff();
  };

  // staggered schedule: logits of the last fragment computed and not yet
  // reduced (fragment NFQ-1 of the previous subtile when a subtile starts)
  f32x16 pend;
#pragma unroll
  for (int a = 0; a < 16; ++a) pend[a] = -__builtin_inff();

  // one 32-key subtile
  auto subtile = [&](const uint16_t* sb, bool masked, int seg, int kbase, auto sub_tag)
                     __attribute__((always_inline)) {
    constexpr int SUB = decltype(sub_tag)::value;
    bf16x8 ak[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) ak[s] = key_op(sb, s);
    auto frag = [&](auto f_tag) __attribute__((always_inline)) {
      constexpr int f = decltype(f_tag)::value;
      f32x16 c = {};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) c = mfma32(ak[s], qop(f_tag, s), c);
      // the pending fragment belongs to the previous subtile for f = 0: it
      // closes a tile when that subtile was the tile's last
      constexpr bool FOLD = f == 0 ? SUB == 0 : SUB == C::NSUB - 1;
      reduce_t(pend, std::integral_constant<int, (f + NFQ - 1) % NFQ>{},
               std::integral_constant<bool, FOLD>{});
      if (masked) mask(c, f, seg, kbase);
      pend = c;
      // keep the next fragment's work from being hoisted into this one
      __builtin_amdgcn_sched_barrier(0);
    };
    frag(std::integral_constant<int, 0>{});
    if constexpr (NFQ > 1) frag(std::integral_constant<int, 1>{});
    if constexpr (NFQ > 2) frag(std::integral_constant<int, 2>{});
    if constexpr (NFQ > 3) frag(std::integral_constant<int, 3>{});
  };

  // tile t sits in buffer BUF: prefetch t+1 into the other buffer, consume
  // t, then wait for the prefetch and publish it with one barrier
  auto step = [&](int t, auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (t + 1 < T) issue_tile(t + 1, BUF ^ 1);
    const int seg = t < T0 ? 0 : 1;
    const int key0 = (seg == 0 ? t : t - T0) * C::KT;
    const bool masked = seg == 0 ? (key0 + C::KT > n_c)
                                 : (key0 + C::KT - 1 > pos_min || key0 + C::KT > n_in);
    const uint16_t* sb = sk + BUF * TL::ELEMS;
    // one copy of the tile loop: the mask is applied under a uniform branch
    static_for<C::NSUB>([&](auto sub_tag) __attribute__((always_inline)) {
      constexpr int sub = decltype(sub_tag)::value;
      subtile(sb + sub * 32 * D, masked, seg, key0 + sub * 32, sub_tag);
    });
    wait_all_mem();
    __syncthreads();
  };

  issue_tile(0, 0);
  wait_all_mem();
  __syncthreads();
  int t = 0;
  for (; t + 1 < Tw; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < Tw) {
    step(t, std::integral_constant<int, 0>{});
    ++t;
  }
  // tiles past this wave's rows: only its share of the loads and the barriers
  for (; t < T; ++t) {
    if (t + 1 < T) issue_tile(t + 1, (t & 1) ^ 1);
    wait_all_mem();
    __syncthreads();
  }
  reduce_t(pend, std::integral_constant<int, NFQ - 1>{}, std::true_type{});
#pragma unroll
  for (int f = 0; f < NFQ; ++f) kahan_add(tp[f], f);   // (0 after whole tiles)

  // merge the two half-waves that hold the same query, then store
#pragma unroll
  for (int f = 0; f < NFQ; ++f) {
    const float own = sum[f] - comp[f];
    const float nmo = __shfl_xor(nm[f], 32);
    const float so = __shfl_xor(own, 32);
    const float nM = __builtin_fminf(nm[f], nmo);  // -(row max) * c2
    const float S = own * fast_exp2(nM - nm[f]) + so * fast_exp2(nM - nmo);
    // row max * scale = -nM * ln 2 (c2 = scale * log2 e)
    const float val = __builtin_fmaf(-nM, kLn2, __logf(S));
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
