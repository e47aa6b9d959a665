// Pieces shared by the persistent slab kernels for bf16, d_h = 64 and short
// sequences (N <= 256): LDS row layout, fragment loads, the four-lane dot
// product and the per-head distance records.
//
// Lanes.  Four lanes own a row (lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave);
// each holds 16 of its 64 elements, so v_permlane32_swap and
// v_permlane16_swap sums complete a dot product.
//
// LDS rows.  bf16 rows take 144 bytes and fp32 rows 272 bytes (an odd
// number of 16-byte units); a lane's 16 elements are chunks 2 p, 2 p + 1
// (bf16) or 4 p .. 4 p + 3 (fp32) of its row for lane part p.  Measured on
// gfx950 (64 banks), a ds_read_b128 serves the two 32-lane halves of a wave
// separately and, within a half, the lane quads whose index has even
// popcount ({0-3, 12-15, 20-23, 24-27}) together and the odd ones together.
// With part = (l / 16) xor parity((l % 16) / 4) for lane l (the row's four
// lanes still hold four different parts), every such group of an fp32 read
// and of a bf16 read hits 16 distinct 16-byte bank groups for any first row:
// no conflicts for either stride, found by exhaustive search.
#pragma once

#include "fib_offsets.h"
#include "kernel_common.h"
#include "launch.h"

#include <algorithm>
#include <cstring>

namespace fibatt {
namespace slab {

constexpr int kMaxRows = 256;        // rows a workgroup covers (16 waves x 16)
constexpr int kMaxPos = 12;          // positive distances below 256: at most 1,2,3,5,...,233
constexpr int kBf16Stride = 144;     // bytes per bf16 row of 64 in LDS (128 + 16)
constexpr int kF32Stride = 272;      // bytes per fp32 row of 64 in LDS (256 + 16)
constexpr int kRowBytes = 128;       // bf16 row of 64 elements in HBM

// Byte offset of 16-byte chunk c of LDS row r.
__device__ __forceinline__ int b16_chunk(int r, int c) { return __umul24(r, kBf16Stride) + c * 16; }
__device__ __forceinline__ int f32_chunk(int r, int c) { return __umul24(r, kF32Stride) + c * 16; }

// Part (which 16 of the 64 elements) lane l of a wave works on.
__device__ __forceinline__ int lane_part(int lane) {
  return ((lane >> 4) & 3) ^ (((lane >> 2) ^ (lane >> 3)) & 1);
}

// Sum of x over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row r clamped into [0, N - 1] (one v_med3_i32; the compiler would emit a
// max and a min).
__device__ __forceinline__ int clamp_row(int r, int N) {
  int c;
  asm("v_med3_i32 %0, %1, 0, %2" : "=v"(c) : "v"(r), "s"(N - 1));
  return c;
}

// First product of an accumulation chain: v_dot2_f32_bf16 with an inline
// zero addend (the builtin with a literal 0 would add a register move).
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---- Four lanes per row (1024-thread kernels) ----------------------------

// Sum of x over the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float quad_sum(float x) {
  const float y = pair_sum(x);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Byte offset of a shifted row fragment: base + delta clamped into [lo, hi]
// (the lane's fragment of the slab's first and last rows).  One asm block:
// the add and the clamp take two VALU instructions.
__device__ __forceinline__ int shifted_off(int base, int delta, int lo, int hi) {
  int c;
  asm("v_add_u32 %0, %1, %2\n\tv_med3_i32 %0, %0, %3, %4"
      : "=&v"(c)
      : "s"(delta), "v"(base), "v"(lo), "v"(hi));
  return c;
}

// LDS byte address of a pointer into LDS.
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ int lds_addr(const char* p) {
  return static_cast<int>(reinterpret_cast<uintptr_t>((lds_cchar*)p));
}

// LDS addresses of this lane's fragment of its own row and of the slab's
// first and last rows, for rows of `stride` bytes starting at `region` and
// lanes that read `frag` bytes at `frag * part`.
struct RowSpan {
  int base, lo, hi;
  __device__ __forceinline__ RowSpan(const char* region, int stride, int frag, int part, int row,
                                     int N)
      : base(lds_addr(region) + frag * part + row * stride),
        lo(lds_addr(region) + frag * part),
        hi(lds_addr(region) + frag * part + (N - 1) * stride) {}
  __device__ __forceinline__ int at(int delta) const { return shifted_off(base, delta, lo, hi); }
};

// This lane's quarter (16 bf16 = 32 bytes) of bf16 LDS row r; `base` already
// points at the lane's part of row 0 (array base + 32 p).
__device__ __forceinline__ void load_bf16_q(const char* base, int r, u32x4 (&f)[2]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(base + __umul24(r, kBf16Stride));
  f[0] = q[0];
  f[1] = q[1];
}

// This lane's quarter (16 fp32 = 64 bytes) of fp32 LDS row r; `base` already
// points at the lane's part of row 0 (array base + 64 p).
__device__ __forceinline__ void load_f32_q(const char* base, int r, u32x4 (&f)[4]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(base + __umul24(r, kF32Stride));
#pragma unroll
  for (int t = 0; t < 4; ++t) f[t] = q[t];
}

// The same fragments at an LDS byte address.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ void load_bf16_at(int addr, u32x4 (&f)[2]) {
  lds_u32x4* q = (lds_u32x4*)static_cast<uintptr_t>(static_cast<uint32_t>(addr));
  f[0] = q[0];
  f[1] = q[1];
}
__device__ __forceinline__ void load_f32_at(int addr, u32x4 (&f)[4]) {
  lds_u32x4* q = (lds_u32x4*)static_cast<uintptr_t>(static_cast<uint32_t>(addr));
#pragma unroll
  for (int t = 0; t < 4; ++t) f[t] = q[t];
}

// This lane's part of the dot product of two bf16 rows (16 elements),
// accumulated in fp32.
__device__ __forceinline__ float dot_part(const uint32_t (&a)[8], const u32x4 (&b)[2]) {
  const uint32_t bw[8] = {b[0].x, b[0].y, b[0].z, b[0].w, b[1].x, b[1].y, b[1].z, b[1].w};
  float acc[2] = {dot2_first(a[0], bw[0]), dot2_first(a[1], bw[1])};
#pragma unroll
  for (int u = 2; u < 8; ++u)
    acc[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[u]),
                                                 __builtin_bit_cast(bf16x2_t, bw[u]), acc[u & 1],
                                                 false);
  return acc[0] + acc[1];
}

// Full 64-element dot product of two bf16 rows split over the row's four
// lanes, accumulated in fp32.
__device__ __forceinline__ float dot_q(const uint32_t (&a)[8], const u32x4 (&b)[2]) {
  return quad_sum(dot_part(a, b));
}

// Transposed reduction over the row's four lanes: x[j] holds this lane's
// partial sum of quantity j; the result is the full sum of quantity
// slot = (lane / 16) % 4.  Three swaps and three adds reduce four
// quantities (a plain quad_sum per quantity would take eight of each).
__device__ __forceinline__ int quad_slot(int lane) { return (lane >> 4) & 3; }

__device__ __forceinline__ float reduce4(const float (&x)[4]) {
  // Across lane halves: the low half keeps quantities 0 and 1, the high
  // half 2 and 3.
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]),
                                                  false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]),
                                                  false, false);
  const float t0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float t1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  // Across 16-lane rows: even rows keep t0, odd rows t1.
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(t0), __float_as_uint(t1), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The inverse gather: x is this lane's value of quantity quad_slot(lane);
// afterwards every lane of the row holds all four (y[j] = quantity j).
__device__ __forceinline__ void gather4(float x, float (&y)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);  // a[0]: slots 0/1, a[1]: slots 2/3
  const auto lo = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
  y[0] = __uint_as_float(lo[0]);
  y[1] = __uint_as_float(lo[1]);
  y[2] = __uint_as_float(hi[0]);
  y[3] = __uint_as_float(hi[1]);
}

// Maximum of x over the four lanes of a row.
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// acc += p * x for this lane's 16 fp32 elements.
__device__ __forceinline__ void axpy_q(float (&acc)[16], float p, const u32x4 (&x)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc[4 * t + 0] = __builtin_fmaf(p, __uint_as_float(x[t].x), acc[4 * t + 0]);
    acc[4 * t + 1] = __builtin_fmaf(p, __uint_as_float(x[t].y), acc[4 * t + 1]);
    acc[4 * t + 2] = __builtin_fmaf(p, __uint_as_float(x[t].z), acc[4 * t + 2]);
    acc[4 * t + 3] = __builtin_fmaf(p, __uint_as_float(x[t].w), acc[4 * t + 3]);
  }
}

// Ascending positive distances of a head, one byte each in three words
// (wave-uniform, so extraction is scalar arithmetic).
struct Dist {
  uint32_t w0, w1, w2;
  __device__ __forceinline__ int at(int i) const {
    const uint32_t w = i < 4 ? w0 : (i < 8 ? w1 : w2);
    return static_cast<int>((w >> (8 * (i & 3))) & 0xffu);
  }
  // Whether j is one of the first n (wave-uniform) distances.
  __device__ __forceinline__ bool has(int j, int n) const {
    bool found = false;
    for (int i = 0; i < n; ++i) found |= at(i) == j;
    return found;
  }
  // Position of distance j among the first n, or -1.
  __device__ __forceinline__ int index(int j, int n) const {
    int k = -1;
    for (int i = 0; i < n; ++i) k = at(i) == j ? i : k;
    return k;
  }
};

// Per-head record handed to the kernels in their arguments: bytes 0..11 are
// the ascending positive distances, byte 12 their count, byte 13 whether 0
// is a distance.  Sixteen bytes per head.
// Host: the record of every head h < H (zero for h >= H, up to MH).  Returns
// false when a head has more positive distances than kMaxPos (or N > 256).
inline bool pack_records(const Problem& p, u32x4* rec, int MH) {
  if (p.N > kMaxRows) return false;
  for (int h = 0; h < MH; ++h) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (h < p.H) {
      int32_t dist[kMaxOffsets];
      const int n = head_distances(p, h, dist);
      if (n > kMaxOffsets) return false;
      int c = 0;
      bool has0 = false;
      for (int i = 0; i < n; ++i) {
        if (dist[i] == 0) {
          has0 = true;
          continue;
        }
        if (c == kMaxPos) return false;
        w[c >> 2] |= static_cast<uint32_t>(dist[i]) << (8 * (c & 3));
        ++c;
      }
      w[3] |= static_cast<uint32_t>(c) | (has0 ? 0x100u : 0u);
    }
    rec[h] = u32x4{w[0], w[1], w[2], w[3]};
  }
  return true;
}

inline bool records_fit(const Problem& p) {
  u32x4 tmp[kMaxHeads];
  return p.H <= kMaxHeads && pack_records(p, tmp, p.H);
}

// Row blocks.  A workgroup's 16 waves each take one block of 16 rows, and
// wave w runs on SIMD w mod 4, so the four SIMDs share the rows of a slab.
// Blocks near either end of the sequence have fewer in-range distances than
// the middle ones; with 13 blocks (N = 197), say, one SIMD gets four of them
// and the other three get three.  plan_blocks picks which block each wave
// takes so that, summed over the heads, the busiest SIMD has as little work
// as a move-and-swap local search finds (from the plain block = wave
// assignment and from a greedy largest-first one).  Four bits per wave;
// blocks past the sequence mark idle waves.
namespace plan_detail {
constexpr int kBlocks = 16;
constexpr int kSimds = 4;
constexpr int kBlockFixed = 3;  // per-block work besides the distances, in distance steps

struct Plan {
  int n[kSimds];
  int8_t b[kSimds][4];
};

inline long plan_score(const Plan& g, const int (*cost)[kBlocks], int H) {
  long s = 0;
  for (int h = 0; h < H; ++h) {
    int m = 0;
    for (int i = 0; i < kSimds; ++i) {
      int l = 0;
      for (int j = 0; j < g.n[i]; ++j) l += cost[h][g.b[i][j]];
      m = l > m ? l : m;
    }
    s += m;
  }
  return s;
}

// Moves of one block to another SIMD and swaps of two blocks, while any
// lowers the score.
inline long plan_improve(Plan& g, const int (*cost)[kBlocks], int H) {
  long best = plan_score(g, cost, H);
  for (bool changed = true; changed;) {
    changed = false;
    for (int s1 = 0; s1 < kSimds; ++s1)
      for (int s2 = 0; s2 < kSimds; ++s2) {
        if (s1 == s2) continue;
        for (int i = 0; i < g.n[s1]; ++i)
          for (int j = 0; j <= g.n[s2]; ++j) {
            Plan t = g;
            if (j < g.n[s2]) {  // swap
              const int8_t x = t.b[s1][i];
              t.b[s1][i] = t.b[s2][j];
              t.b[s2][j] = x;
            } else {  // move
              if (t.n[s2] == 4) continue;
              t.b[s2][t.n[s2]++] = t.b[s1][i];
              t.b[s1][i] = t.b[s1][--t.n[s1]];
            }
            const long sc = plan_score(t, cost, H);
            if (sc < best) {
              best = sc;
              g = t;
              changed = true;
            }
          }
      }
  }
  return best;
}
}  // namespace plan_detail

inline uint64_t plan_blocks(int N, int H, const u32x4* rec) {
  using namespace plan_detail;
  const int nb = (N + 15) / 16;
  static thread_local int last_n = -1, last_h = -1;
  static thread_local u32x4 last_rec[kMaxHeads];
  static thread_local uint64_t last_plan = 0;
  if (N == last_n && H == last_h && memcmp(rec, last_rec, sizeof(u32x4) * H) == 0)
    return last_plan;

  int cost[kMaxHeads][kBlocks] = {};
  for (int h = 0; h < H; ++h) {
    const int cnt = static_cast<int>(rec[h].w & 0xffu);
    const uint32_t w[3] = {rec[h].x, rec[h].y, rec[h].z};
    for (int b = 0; b < nb; ++b) {
      const int r0 = 16 * b, rl = r0 + 15 < N ? r0 + 15 : N - 1;
      int c = kBlockFixed;
      for (int i = 0; i < cnt; ++i) {
        const int f = static_cast<int>((w[i >> 2] >> (8 * (i & 3))) & 0xffu);
        c += (r0 + f < N ? 1 : 0) + (f <= rl ? 1 : 0);
      }
      cost[h][b] = c;
    }
  }
  Plan plain = {}, greedy = {};
  for (int b = 0; b < nb; ++b) plain.b[b % kSimds][plain.n[b % kSimds]++] = static_cast<int8_t>(b);
  {
    long tot[kBlocks] = {}, load[kSimds] = {};
    int order[kBlocks];
    for (int b = 0; b < nb; ++b) {
      for (int h = 0; h < H; ++h) tot[b] += cost[h][b];
      order[b] = b;
    }
    std::stable_sort(order, order + nb, [&](int x, int y) { return tot[x] > tot[y]; });
    for (int k = 0; k < nb; ++k) {
      int s = -1;
      for (int i = 0; i < kSimds; ++i)
        if (greedy.n[i] < 4 && (s < 0 || load[i] < load[s])) s = i;
      greedy.b[s][greedy.n[s]++] = static_cast<int8_t>(order[k]);
      load[s] += tot[order[k]];
    }
  }
  const long sp = plan_improve(plain, cost, H);
  const long sg = plan_improve(greedy, cost, H);
  const Plan& g = sg < sp ? greedy : plain;

  uint64_t plan = 0;
  int idle = nb;
  for (int w = 0; w < kBlocks; ++w) {
    const int s = w % kSimds, slot = w / kSimds;
    const int b = slot < g.n[s] ? g.b[s][slot] : idle++;
    plan |= static_cast<uint64_t>(b) << (4 * w);
  }
  last_n = N;
  last_h = H;
  memcpy(last_rec, rec, sizeof(u32x4) * H);
  last_plan = plan;
  return plan;
}

// Compute units of the current device (cached per process).
inline int cu_count() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return cus;
  }();
  return n > 0 ? n : 256;
}

}  // namespace slab
}  // namespace fibatt
