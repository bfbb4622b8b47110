// Device-side helpers shared by the gfx950 kernels of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace kvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;            // MI355X: 8 accelerator dies, 32 CUs each
constexpr float kLn2 = 0.6931471805599453f;

// D += A * B on the 32x32x16 bf16 matrix core op.  Lane l supplies
// A[l % 32][8 * (l / 32) + 0..7] and B[8 * (l / 32) + 0..7][l % 32]; it gets
// back D[8 * (a / 4) + 4 * (l / 32) + a % 4][l % 32] in element a of the
// accumulator, so each lane holds 16 rows of a single output column.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32-row block) of accumulator element a held by lane l.
__device__ __forceinline__ int acc_row(int a, int lane) {
  return 8 * (a >> 2) + 4 * (lane >> 5) + (a & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte load of data read exactly once (streams and gathers): marked
// non-temporal so that it does not displace reused lines in the caches
__device__ __forceinline__ u32x4 ldg16_once(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 16-byte store of data this kernel does not read again: non-temporal
__device__ __forceinline__ void stg16_once(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ u32x4 zero16() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// Workgroups are handed to the 8 dies round-robin (block b runs on die
// b % 8).  Renumber them so each die receives one contiguous range of logical
// ids: neighbouring work (the same head) then shares that die's L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  return xcd * q + (xcd < r ? xcd : r) + bid / kXcds;
}

// A tile of bf16 rows of length D in LDS, 32 KB per buffer, filled straight
// from global memory by 16-byte LDS-DMA loads (global_load_lds_dwordx4: each
// wave instruction writes 64 x 16 B contiguously, so no register staging and
// no LDS store instructions are needed).
//
// Layout: row r occupies elements [r*D, (r+1)*D); its 16-byte chunk c is
// stored in chunk slot c ^ swz(r).  The matrix-operand reads take 16 bytes of
// one row per lane, 32 rows at a time; the XOR spreads 16 consecutive rows of
// the same chunk over distinct LDS banks, so those reads are conflict-free
// without padding (padding is impossible with contiguous DMA writes).
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWS = 16384 / D;            // 32 KB of bf16 per buffer
  static constexpr int ELEMS = ROWS * D;
  static constexpr int LOADS = ROWS * CPR / 256;    // 16-B loads per thread (256 threads)
  __device__ static __forceinline__ int swz(int r) {
    return D == 64 ? ((r >> 1) & 7) : (r & 15);
  }
  // element offset, within a tile, of the load slot (i, tid) and the global
  // element offset (relative to the tile's first row) it must fetch
  __device__ static __forceinline__ int src_rel(int i, int tid) {
    const int s = i * 256 + tid;
    const int r = s / CPR, p = s % CPR;
    return r * D + ((p ^ swz(r)) * 8);
  }
  __device__ static __forceinline__ int src_row(int i, int tid) {
    return (i * 256 + tid) / CPR;
  }
  // element offset of the 16 B lane l reads for k-step s of a 32-row block
  // starting at row 0 (add 32 * D per further block)
  __device__ static __forceinline__ int read_off(int lane, int s) {
    const int r = lane & 31;
    const int c = 2 * s + (lane >> 5);
    return r * D + ((c ^ swz(r)) * 8);
  }
  // The same offset from two per-lane values, so that no table of KS offsets
  // stays live: with chunk c = 2 s + h (h = lane / 32) and any swizzle value
  // w, c ^ w = 2 (s ^ (w >> 1)) + (h ^ (w & 1)), hence
  //   read_off(lane, s) = read_base(lane) + 16 * (s ^ read_x(lane)).
  __device__ static __forceinline__ int read_base(int lane) {
    const int r = lane & 31;
    return r * D + 8 * ((lane >> 5) ^ (swz(r) & 1));
  }
  __device__ static __forceinline__ int read_x(int lane) { return swz(lane & 31) >> 1; }
  // src_rel(i, tid) = src_rel(i & 1, tid) + (i & ~1) * 2048: one slot is 256
  // chunks = 2048 elements, and two slots span 4096 / D >= 16 rows, a whole
  // number of swizzle periods (16 rows), so two per-thread offsets serve
  // every load of a tile.
  __device__ static __forceinline__ int src_rel_from(const int (&rel01)[2], int i) {
    return rel01[i & 1] + (i & ~1) * 2048;
  }
};

// 16-byte global -> LDS copy; `lds` must be the same for the whole wave (the
// lane's data lands at lds + 16 * lane).
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds) {
  __builtin_amdgcn_global_load_lds(gsrc, lds, 16, 0, 0);
}
// 4-byte global -> LDS copy; the lane's data lands at lds + 4 * lane.
__device__ __forceinline__ void lds_dma4(const void* gsrc, void* lds) {
  __builtin_amdgcn_global_load_lds(gsrc, lds, 4, 0, 0);
}

// Wait for this wave's outstanding memory operations (incl. LDS-DMA).
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace kvq
