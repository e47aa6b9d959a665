// Pieces shared by the long-sequence tile kernels (bf16, d_h = 64 or 128).
// A lane quad owns 64 elements of a row: lane p of the quad works on the
// 8-element groups p and p + 4 of them, so a quad reads or writes 64
// contiguous bytes per instruction.  A row of d_h = 64 is one quad (16 rows
// per wave); a row of 128 is two quads 32 lanes apart, one per half (8 rows
// per wave).  Sums over a quad use DPP quad permutations, and the two halves
// of a 128-wide row are joined with v_permlane32_swap.  Workgroups of 4 waves
// take tiles of 64 or 32 rows, numbered slab by slab and dealt to the XCDs in
// contiguous ranges (workgroup b runs on XCD b mod 8) so that the tiles of a
// slab share an L2.
#pragma once

#include "slab_bf16_common.h"

namespace fibatt {
namespace tile {

constexpr int kTileThreads = 256;  // 4 waves
constexpr int kXcds = 8;

// NQ quads per row (d_h = 64 NQ).
template <int NQ>
struct Geo {
  static constexpr int kRowB = 128 * NQ;              // bf16 row bytes
  static constexpr int kRows = kTileThreads / 4 / NQ;  // rows per tile
  static constexpr int kD = 64 * NQ;
};

// DPP quad permutations: lane i of each quad reads lane P[i].
constexpr int kSwap1 = 0xB1;  // [1, 0, 3, 2]
constexpr int kSwap2 = 0x4E;  // [2, 3, 0, 1]

template <int CTRL>
__device__ __forceinline__ float qperm(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum and maximum of x over the lane quad.
__device__ __forceinline__ float quad_sum4(float x) {
  x += qperm<kSwap1>(x);
  return x + qperm<kSwap2>(x);
}
__device__ __forceinline__ float quad_max4(float x) {
  x = fmaxf(x, qperm<kSwap1>(x));
  return fmaxf(x, qperm<kSwap2>(x));
}

// Transposed reduction over the quad: x[j] is this lane's partial sum of
// quantity j; the result is the full sum of quantity lane % 4.  Each round
// keeps half of the quantities and sends the other half to the partner lane.
__device__ __forceinline__ float reduce4q(const float (&x)[4], bool b0, bool b1) {
  const float u0 = (b0 ? x[1] : x[0]) + qperm<kSwap1>(b0 ? x[0] : x[1]);
  const float u1 = (b0 ? x[3] : x[2]) + qperm<kSwap1>(b0 ? x[2] : x[3]);
  return (b1 ? u1 : u0) + qperm<kSwap2>(b1 ? u0 : u1);
}

// x summed with the other half of a 128-wide row, which sits 32 lanes away
// (for partial dot products; values both halves already share need no join).
template <int NQ>
__device__ __forceinline__ float halves_sum(float x) {
  if constexpr (NQ == 2) return slab::pair_sum(x);
  return x;
}
// Row (within a tile) and half of lane `tid`: a wave holds 16 rows of
// d_h = 64 (quad q = lane / 4 is row q), or 8 rows of d_h = 128 with the
// first halves in lanes 0-31 and the second halves in lanes 32-63.
template <int NQ>
__device__ __forceinline__ int tile_row(int tid) {
  if constexpr (NQ == 2) return (tid >> 6) * 8 + ((tid & 31) >> 2);
  return tid >> 2;
}
template <int NQ>
__device__ __forceinline__ int row_half(int tid) {
  if constexpr (NQ == 2) return (tid >> 5) & 1;
  return 0;
}

// y[j] = x of lane j of the quad.
__device__ __forceinline__ void gather4q(float x, float (&y)[4]) {
  y[0] = qperm<0x00>(x);
  y[1] = qperm<0x55>(x);
  y[2] = qperm<0xAA>(x);
  y[3] = qperm<0xFF>(x);
}

// This lane's 16 elements (groups p and p + 4) of a bf16 row; rowp already
// points at byte 16 p of the row.
__device__ __forceinline__ void load_row_q(const char* rowp, u32x4 (&f)[2]) {
  f[0] = *reinterpret_cast<const u32x4*>(rowp);
  f[1] = *reinterpret_cast<const u32x4*>(rowp + 64);
}

// acc += p * x for this lane's 16 bf16 elements (widened to fp32).
__device__ __forceinline__ void axpy_bf16(float (&acc)[16], float p, const u32x4 (&x)[2]) {
  const uint32_t w[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    acc[2 * u] = __builtin_fmaf(p, __uint_as_float(w[u] << 16), acc[2 * u]);
    acc[2 * u + 1] = __builtin_fmaf(p, __uint_as_float(w[u] & 0xffff0000u), acc[2 * u + 1]);
  }
}

// acc_a += pa * x and acc_b += pb * x for this lane's 16 bf16 elements
// (each widened to fp32 once).
__device__ __forceinline__ void axpy2_bf16(float (&acc_a)[16], float pa, float (&acc_b)[16],
                                           float pb, const u32x4 (&x)[2]) {
  const uint32_t w[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float lo = __uint_as_float(w[u] << 16), hi = __uint_as_float(w[u] & 0xffff0000u);
    acc_a[2 * u] = __builtin_fmaf(pa, lo, acc_a[2 * u]);
    acc_a[2 * u + 1] = __builtin_fmaf(pa, hi, acc_a[2 * u + 1]);
    acc_b[2 * u] = __builtin_fmaf(pb, lo, acc_b[2 * u]);
    acc_b[2 * u + 1] = __builtin_fmaf(pb, hi, acc_b[2 * u + 1]);
  }
}

// acc += sum_j c_j x_j over a group of four bf16 fragments x_j (this lane's
// 16 elements each), with the coefficients packed as bf16 pairs c01 = (c_0,
// c_1) and c23 = (c_2, c_3).  Element e of two fragments is interleaved
// into one bf16 pair (v_perm_b32) and v_dot2_f32_bf16 adds both products
// to the fp32 accumulator: 16 instructions per fragment instead of 32 for
// widening and fp32 FMAs.  The coefficients lose their low mantissa bits
// (relative 2^-9), as a bf16 matrix-core product would.
__device__ __forceinline__ void axpy4_dot2(float (&acc)[16], uint32_t c01, uint32_t c23,
                                           const u32x4 (&x)[4][2]) {
  constexpr uint32_t kLo = 0x05040100u;  // (a.lo, b.lo): bytes 0, 1 of a, then of b
  constexpr uint32_t kHi = 0x07060302u;  // (a.hi, b.hi)
  const bf16x2_t p01 = __builtin_bit_cast(bf16x2_t, c01);
  const bf16x2_t p23 = __builtin_bit_cast(bf16x2_t, c23);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t a = x[0][u >> 2][u & 3], b = x[1][u >> 2][u & 3];
    const uint32_t c = x[2][u >> 2][u & 3], d = x[3][u >> 2][u & 3];
    float lo = __builtin_amdgcn_fdot2_f32_bf16(
        p01, __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b, a, kLo)), acc[2 * u], false);
    float hi = __builtin_amdgcn_fdot2_f32_bf16(
        p01, __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b, a, kHi)), acc[2 * u + 1], false);
    lo = __builtin_amdgcn_fdot2_f32_bf16(
        p23, __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(d, c, kLo)), lo, false);
    hi = __builtin_amdgcn_fdot2_f32_bf16(
        p23, __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(d, c, kHi)), hi, false);
    acc[2 * u] = lo;
    acc[2 * u + 1] = hi;
  }
}

// Workgroup b's tile index (-1 for none), b running on XCD x = b mod 8.
//  * Small slabs (per_xcd > 0): XCD x takes the contiguous range
//    [x * per_xcd, (x + 1) * per_xcd) of all tiles, so a slab's tiles share
//    one L2.
//  * Large slabs (chunk > 0): every slab's tiles are cut into 8 contiguous
//    chunks of `chunk` tiles; XCD x takes chunk x of slab 0, then of slab 1,
//    and so on.  All XCDs work on one slab at a time (its K and V stay in the
//    Infinity Cache) while each keeps its own row window in its L2.
__device__ __forceinline__ int tile_of_block(int per_xcd, int chunk, int tiles) {
  const int x = static_cast<int>(blockIdx.x % kXcds);
  const int k = static_cast<int>(blockIdx.x / kXcds);
  if (chunk == 0) return x * per_xcd + k;
  const int slab = k / chunk;
  const int t = x * chunk + (k - slab * chunk);
  return t < tiles ? slab * tiles + t : -1;
}

// Launch shape for `slabs` slabs of `tiles` tiles whose K and V take
// `slab_kv` bytes: the first order above while a slab's K and V fit in half
// an L2 (4 MB per XCD), the second otherwise.  Returns the grid size.
inline long long tile_grid(long long slabs, int tiles, long long slab_kv, int& per_xcd,
                          int& chunk) {
  constexpr long long kHalfL2 = 2ll << 20;
  const long long work = slabs * tiles;
  if (slab_kv <= kHalfL2) {
    chunk = 0;
    per_xcd = static_cast<int>((work + kXcds - 1) / kXcds);
    return static_cast<long long>(per_xcd) * kXcds;
  }
  per_xcd = 0;
  chunk = (tiles + kXcds - 1) / kXcds;
  return slabs * chunk * kXcds;
}

// Signed displacements of the head with the most (2 per positive distance,
// 1 for distance 0).
inline int max_signed(const Problem& p) {
  int best = 0;
  for (int h = 0; h < p.H; ++h) {
    int32_t dist[kMaxOffsets];
    const int n = head_distances(p, h, dist);
    int c = 0;
    for (int i = 0; i < (n < kMaxOffsets ? n : kMaxOffsets); ++i) c += dist[i] == 0 ? 1 : 2;
    best = c > best ? c : best;
  }
  return best;
}

}  // namespace tile
}  // namespace fibatt
