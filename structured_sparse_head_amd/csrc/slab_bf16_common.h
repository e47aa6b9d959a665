// Pieces shared by the persistent slab kernels for bf16, d_h = 64 and short
// sequences (N <= 256): lane layout, LDS row strides, fragment loads, the
// two-lane dot product and the per-head distance records.
//
// Lanes.  Two lanes own a row, each holding 32 of its 64 elements: lanes
// 0-31 of a wave take the first halves of 32 consecutive rows and lanes
// 32-63 the second halves, so one v_permlane32_swap plus one add completes a
// dot product.
//
// LDS strides.  bf16 rows use 144 bytes and fp32 rows 272 bytes, both an odd
// number of 16-byte units.  Measured on gfx950 (64 banks), a ds_read_b128
// serves the two 32-lane halves of a wave separately and, within a half, the
// lane quads whose index has even popcount ({0-3, 12-15, 20-23, 24-27})
// together and the odd ones together.  Each such group reads 16 rows that
// are distinct modulo 16, and an odd stride maps them to 16 distinct 16-byte
// bank groups: no conflicts.
#pragma once

#include "fib_offsets.h"
#include "kernel_common.h"
#include "launch.h"

namespace fibatt {
namespace slab {

constexpr int kThreads = 512;        // 8 waves; 256 rows at 2 lanes per row
constexpr int kMaxRows = kThreads / 2;
constexpr int kMaxPos = 12;          // positive distances below 256: at most 1,2,3,5,...,233
constexpr int kBf16Stride = 144;     // bytes per bf16 row of 64 in LDS (128 + 16)
constexpr int kF32Stride = 272;      // bytes per fp32 row of 64 in LDS (256 + 16)
constexpr int kRowBytes = 128;       // bf16 row of 64 elements in HBM
constexpr int kChunksPerThread = kMaxRows * (kRowBytes / 16) / kThreads;  // 4

// Sum of x over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int clamp_row(int r, int N) { return r < 0 ? 0 : (r >= N ? N - 1 : r); }

// This lane's half (32 bf16 = 64 bytes) of LDS row r.
__device__ __forceinline__ void load_bf16_half(const char* base, int r, int part, u32x4 (&f)[4]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + __umul24(r, kBf16Stride) + part * 64);
#pragma unroll
  for (int t = 0; t < 4; ++t) f[t] = p[t];
}

// This lane's half (32 fp32 = 128 bytes) of LDS row r.
__device__ __forceinline__ void load_f32_half(const char* base, int r, int part, u32x4 (&f)[8]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + __umul24(r, kF32Stride) + part * 128);
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = p[t];
}

__device__ __forceinline__ void unpack_words(const u32x4 (&x)[4], uint32_t (&w)[16]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    w[4 * t + 0] = x[t].x;
    w[4 * t + 1] = x[t].y;
    w[4 * t + 2] = x[t].z;
    w[4 * t + 3] = x[t].w;
  }
}

// First product of an accumulation chain: v_dot2_f32_bf16 with an inline
// zero addend (the builtin with a literal 0 would add a register move).
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Full 64-element dot product of two bf16 rows split over the lane pair,
// accumulated in fp32.
__device__ __forceinline__ float dot_bf16(const uint32_t (&a)[16], const u32x4 (&b)[4]) {
  float acc[4] = {dot2_first(a[0], b[0].x), dot2_first(a[1], b[0].y), dot2_first(a[2], b[0].z),
                  dot2_first(a[3], b[0].w)};
#pragma unroll
  for (int t = 1; t < 4; ++t) {
    const uint32_t bw[4] = {b[t].x, b[t].y, b[t].z, b[t].w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[4 * t + u]),
                                               __builtin_bit_cast(bf16x2_t, bw[u]), acc[u], false);
  }
  return pair_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// acc += p * x for this lane's 32 fp32 elements.
__device__ __forceinline__ void axpy_f32(float (&acc)[32], float p, const u32x4 (&x)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    acc[4 * t + 0] = __builtin_fmaf(p, __uint_as_float(x[t].x), acc[4 * t + 0]);
    acc[4 * t + 1] = __builtin_fmaf(p, __uint_as_float(x[t].y), acc[4 * t + 1]);
    acc[4 * t + 2] = __builtin_fmaf(p, __uint_as_float(x[t].z), acc[4 * t + 2]);
    acc[4 * t + 3] = __builtin_fmaf(p, __uint_as_float(x[t].w), acc[4 * t + 3]);
  }
}

// acc += p * x for this lane's 32 bf16 elements (widened exactly to fp32).
__device__ __forceinline__ void axpy_bf16(float (&acc)[32], float p, const u32x4 (&x)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t w[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[8 * t + 2 * u] = __builtin_fmaf(p, __uint_as_float(w[u] << 16), acc[8 * t + 2 * u]);
      acc[8 * t + 2 * u + 1] =
          __builtin_fmaf(p, __uint_as_float(w[u] & 0xffff0000u), acc[8 * t + 2 * u + 1]);
    }
  }
}

// Writes this lane's 32 bf16 elements (packed in w) as fp32 to an LDS row.
__device__ __forceinline__ void store_f32_half_from_bf16(char* base, int r, int part,
                                                         const uint32_t (&w)[16]) {
  u32x4* p = reinterpret_cast<u32x4*>(base + r * kF32Stride + part * 128);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    p[t] = u32x4{w[2 * t] << 16, w[2 * t] & 0xffff0000u, w[2 * t + 1] << 16,
                 w[2 * t + 1] & 0xffff0000u};
}

// Writes this lane's 32 fp32 elements times `scale` to a global row.
__device__ __forceinline__ void store_f32_half_global(float* row, int part, const float (&x)[32],
                                                      float scale) {
  float4* p = reinterpret_cast<float4*>(row) + part * 8;
#pragma unroll
  for (int t = 0; t < 8; ++t)
    p[t] = make_float4(x[4 * t] * scale, x[4 * t + 1] * scale, x[4 * t + 2] * scale,
                       x[4 * t + 3] * scale);
}

// ---- Four lanes per row (1024-thread kernels) ----------------------------

// Sum of x over the four lanes of a row (l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float quad_sum(float x) {
  const float y = pair_sum(x);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// This lane's quarter (16 bf16 = 32 bytes) of a bf16 LDS row.
__device__ __forceinline__ void load_bf16_q(const char* base, int r, int part, u32x4 (&f)[2]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + __umul24(r, kBf16Stride) + part * 32);
  f[0] = p[0];
  f[1] = p[1];
}

// This lane's quarter (16 fp32 = 64 bytes) of an fp32 LDS row.
__device__ __forceinline__ void load_f32_q(const char* base, int r, int part, u32x4 (&f)[4]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base + __umul24(r, kF32Stride) + part * 64);
#pragma unroll
  for (int t = 0; t < 4; ++t) f[t] = p[t];
}

// Full 64-element dot product of two bf16 rows split over the row's four
// lanes, accumulated in fp32.
__device__ __forceinline__ float dot_q(const uint32_t (&a)[8], const u32x4 (&b)[2]) {
  float acc[4] = {dot2_first(a[0], b[0].x), dot2_first(a[1], b[0].y), dot2_first(a[2], b[0].z),
                  dot2_first(a[3], b[0].w)};
  const uint32_t bw[4] = {b[1].x, b[1].y, b[1].z, b[1].w};
#pragma unroll
  for (int u = 0; u < 4; ++u)
    acc[u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[4 + u]),
                                             __builtin_bit_cast(bf16x2_t, bw[u]), acc[u], false);
  return quad_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
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
};

// Per-head record handed to the kernels in their arguments: bytes 0..11 are
// the ascending positive distances, byte 12 their count, byte 13 whether 0
// is a distance.  Sixteen bytes per head.
struct HeadRecord {
  int pos[kMaxPos];
  int npos;
  bool has0;
};

__device__ __forceinline__ HeadRecord unpack_record(const u32x4& rec) {
  HeadRecord r;
  const uint32_t w[4] = {rec.x, rec.y, rec.z, rec.w};
  r.npos = static_cast<int>(w[3] & 0xffu);
  r.has0 = ((w[3] >> 8) & 0xffu) != 0;
#pragma unroll
  for (int i = 0; i < kMaxPos; ++i) r.pos[i] = static_cast<int>((w[i >> 2] >> (8 * (i & 3))) & 0xffu);
  return r;
}

// Host: the record of every head h < H (zero for h >= H, up to MH).  Returns
// false when a head has more positive distances than kMaxPos (or N > 256).
inline bool pack_records(const Problem& p, u32x4* rec, int MH) {
  if (p.N > kMaxRows) return false;
  for (int h = 0; h < MH; ++h) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (h < p.H) {
      int32_t dist[kMaxOffsets];
      const int n = fib_offsets_gen(p.heads.a[h], p.heads.b[h], p.heads.lim[h], dist, kMaxOffsets);
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
