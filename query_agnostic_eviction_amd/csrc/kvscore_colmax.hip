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
//  * A workgroup of 4 waves owns 512 cached keys (4 fragments of 32 per
//    wave, kept in registers as the B operand; 256 keys in 2 fragments at
//    d = 256, where a fragment takes twice the registers); it sweeps all
//    G * n_in query rows of its head in 32 KB tiles (16384 / d rows),
//    double-buffered and filled by LDS-DMA straight from HBM together with
//    the rows' lse.  Every operand read from LDS feeds four matrix ops.
//  * The accumulator of each 32x32x16 product is seeded with -lse / scale of
//    its rows, so the matrix op itself yields q.k - lse / scale; each lane
//    holds 16 rows of one key and keeps a lane-local running max (max3 on
//    the accumulators, built without NaN semantics: inputs are finite).
//  * Rows are never masked: the last tile is shifted back to end at the last
//    row, and rows it shares with the tile before are simply seen twice,
//    which leaves a maximum unchanged.  Together with per-lane operand
//    offsets formed on the fly this keeps four fragments per wave within
//    the registers of two waves per SIMD.
//  * Within a tile the query-operand reads from LDS run one k-step ahead of
//    the products, and each subtile's seed is formed while the previous
//    subtile's products run (a tile's first subtile waits: its data arrives
//    with the tile).  The compiler's waits on LDS reads drain every
//    outstanding read, so where a work item's query stream is moderate each
//    read is also pinned after its k-step's first product, which keeps it
//    off the wait for the current operand (PIN below).
//  * No atomics: each workgroup owns its columns, writes them once, and the
//    result is independent of scheduling.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int D>
struct ColCfg {
  static constexpr int QT = Tile<D>::ROWS;  // query rows per tile
  static constexpr int NSUB = QT / 32;
  static constexpr int KS = D / 16;
  static constexpr int LSE_LOADS = QT / 64;  // 4-byte DMA instructions per tile
  // cached-key fragments of 32 per wave: each operand read from LDS feeds
  // NF matrix ops
  static constexpr int NF = D == 256 ? 2 : 4;
  static constexpr int KEYS_PER_WG = 4 * NF * 32;
};

// SMALL: fewer rows than one tile (G * n_in < QT); the tile then clamps rows
// past the last one to the last row (duplicates again).
// PIN: each k-step's operand read is pinned after its first product (see the
// tile loop); the launcher sets it where a head's query stream is moderate.
template <int D, bool SMALL, bool PIN>
__global__ __launch_bounds__(256, 2) void colmax_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_ctx,
    const float* __restrict__ lse, float* __restrict__ scores,
    const ScoreShape sh, int wg_per_head, float c2, float inv_scale) {
  using C = ColCfg<D>;
  using TL = Tile<D>;
  constexpr int NF = C::NF;
  __shared__ __attribute__((aligned(1024))) uint16_t sq[2 * TL::ELEMS];
  __shared__ __attribute__((aligned(1024))) float sl[2 * C::QT];

  const int G = sh.G, n_c = sh.n_c, n_in = sh.n_in;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int u = logical / wg_per_head;  // work item: (layer, KV head[, chunk])
  const int j0 = (logical % wg_per_head) * C::KEYS_PER_WG;

  // this wave's key fragments -> registers (B operand layout)
  bf16x8 bk[NF][C::KS];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int key = j0 + 32 * (NF * wave + f) + (lane & 31);
    const bool ok = key < n_c;
    const uint16_t* src = k_ctx + map_offset(sh.k_ctx, u, sh.inner) +
                          (size_t)(ok ? key : 0) * D + 8 * (lane >> 5);
    const uint32_t keep = ok ? 0xffffffffu : 0u;  // keys past n_c read as zeros
#pragma unroll
    for (int s = 0; s < C::KS; ++s) bk[f][s] = as_bf16x8(ldg16(src + 16 * s) & keep);
  }

  const int R = G * n_in;  // flattened (g, i) rows of this head
  const uint16_t* qh = q + map_offset(sh.q, u, sh.inner);
  const float* lh_lse = lse + map_offset(sh.lse, u, sh.inner);
  const int T = (R + C::QT - 1) / C::QT;

  const int rel01[2] = {TL::src_rel(0, tid), TL::src_rel(1, tid)};
  const int rd_base = TL::read_base(lane), rd_x = TL::read_x(lane);

  // LDS-DMA of tile t (query rows and their lse) into buffer `buf`.  The
  // last tile starts at R - QT, so every load is in bounds.
  auto issue_tile = [&](int t, int buf) {
    const int r0 = SMALL ? 0 : min(t * C::QT, R - C::QT);
    const uint16_t* base = qh + (size_t)r0 * D;
    uint16_t* dst = sq + buf * TL::ELEMS + wave * 64 * 8;
    if constexpr (!SMALL) {
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i)
        lds_dma16(base + TL::src_rel_from(rel01, i), dst + i * 256 * 8);
      if (wave < C::LSE_LOADS)
        lds_dma4(lh_lse + r0 + wave * 64 + lane, sl + buf * C::QT + wave * 64);
    } else {
      const int last = R - 1;
#pragma unroll
      for (int i = 0; i < TL::LOADS; ++i) {
        const int r = TL::src_row(i, tid);
        const int rel = TL::src_rel_from(rel01, i) - (r > last ? (r - last) * D : 0);
        lds_dma16(base + rel, dst + i * 256 * 8);
      }
      if (wave < C::LSE_LOADS) {
        const int r = wave * 64 + lane;
        lds_dma4(lh_lse + (r > last ? last : r), sl + buf * C::QT + wave * 64);
      }
    }
  };

  float M[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) M[f] = -__builtin_inff();

  // -lse/scale of the lane's 16 rows of a 32-row subtile: the seed of its
  // products' accumulators
  auto seed = [&](const float* slb) {
    f32x16 init;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(slb + 8 * grp + 4 * (lane >> 5));
#pragma unroll
      for (int e = 0; e < 4; ++e) init[4 * grp + e] = -v[e] * inv_scale;
    }
    return init;
  };
  auto qread = [&](const uint16_t* sb, int s) {
    return *reinterpret_cast<const bf16x8*>(sb + rd_base + 16 * (s ^ rd_x));
  };

  // tile t sits in buffer BUF: prefetch t+1 into the other buffer, consume
  // t, then wait for the prefetch and publish it with one barrier.  Within
  // the tile the operand reads run one k-step ahead of the products, and a
  // subtile's seed is formed while the previous subtile's products run.
  auto step = [&](int t, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (t + 1 < T) issue_tile(t + 1, BUF ^ 1);
    const uint16_t* sb = sq + BUF * TL::ELEMS;
    const float* slb = sl + BUF * C::QT;
    f32x16 init = seed(slb);
    bf16x8 a = qread(sb, 0);
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const uint16_t* sbs = sb + sub * 32 * D;
      f32x16 c[NF];
      f32x16 init_next;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        // With PIN: the first product, then the next operand's read, then
        // the other products.  The wait for an LDS read here drains every
        // outstanding one, so a read issued right before the wait for the
        // current operand is waited for at once; placed after the first
        // product, it is covered by the other three, and the wait before the
        // next k-step drains it alone.
        if constexpr (PIN) {
          c[0] = mfma32(a, bk[0][s], s == 0 ? init : c[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 a_next;
        if (s + 1 < C::KS) a_next = qread(sbs, s + 1);
        else if (sub + 1 < C::NSUB) a_next = qread(sbs + 32 * D, 0);
        if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = PIN ? 1 : 0; f < NF; ++f) c[f] = mfma32(a, bk[f][s], s == 0 ? init : c[f]);
        if (s == C::KS / 2 && sub + 1 < C::NSUB) init_next = seed(slb + (sub + 1) * 32);
        a = a_next;
      }
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          M[f] = max3f(M[f], c[f][4 * g4], max3f(c[f][4 * g4 + 1], c[f][4 * g4 + 2], c[f][4 * g4 + 3]));
      if (sub + 1 < C::NSUB) init = init_next;
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

#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const float mx = __builtin_fmaxf(M[f], __shfl_xor(M[f], 32));
    // the exact score is a probability, so never above 1
    const float sc = __builtin_fminf(fast_exp2(mx * c2), 1.0f);
    const int key = j0 + 32 * (NF * wave + f) + (lane & 31);
    if (lane < 32 && key < n_c) scores[map_offset(sh.scores, u, sh.inner) + key] = sc;
  }
}

// The pinned operand reads make a k-step's products wait less on LDS (about
// 2 % faster, measured on MI355X at 8K, 32K and d = 256 16K contexts), but
// with a long query stream per head (134 MB at a 128K context) the
// workgroups of a head then drift apart over the sweep and read it from HBM
// many times over (13x the traffic, 1.5 % slower).  Pinned up to this many
// bytes of queries per work item; above, the compiler's order.
constexpr long long kPinQueryBytes = 64ll << 20;

template <int D>
hipError_t launch_colmax_d(const uint16_t* q, const uint16_t* k_ctx,
                           const float* lse, float* scores, const ScoreShape& s,
                           hipStream_t stream) {
  constexpr int KPW = ColCfg<D>::KEYS_PER_WG;
  // the last workgroup of a work item is padded (keys past n_c read as zeros
  // and are not stored)
  const int wg_per_head = (s.n_c + KPW - 1) / KPW;
  const long long grid = (long long)s.nheads * wg_per_head;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c2 = s.scale * kLog2e;
  const float inv_scale = (float)(1.0 / (double)s.scale);
  const long long rows = (long long)s.G * s.n_in;
  if (rows < ColCfg<D>::QT)
    hipLaunchKernelGGL((colmax_kernel<D, true, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, k_ctx, lse, scores, s, wg_per_head, c2, inv_scale);
  else if (rows * D * 2 <= kPinQueryBytes)
    hipLaunchKernelGGL((colmax_kernel<D, false, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, k_ctx, lse, scores, s, wg_per_head, c2, inv_scale);
  else
    hipLaunchKernelGGL((colmax_kernel<D, false, false>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, k_ctx, lse, scores, s, wg_per_head, c2, inv_scale);
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
