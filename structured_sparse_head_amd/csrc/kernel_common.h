// Device-side building blocks shared by the forward and backward kernels.
//
// Work decomposition used throughout: a query (or key) row of d_h elements is
// owned by a group of G consecutive lanes; each lane holds a contiguous
// "fragment" of d_h / G elements (a whole number of 16-byte chunks) in
// registers.  Dot products are summed inside the lane, then across the G
// lanes with DPP quad permutes, which never leave a group of 4 (8 for G=8,
// via a half-row mirror).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "problem.h"

namespace fibatt {

using bf16_t = uint16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Geometry of one row split over G lanes.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
struct Geom {
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
  static constexpr int kCPR = kRowBytes / 16;  // 16-byte chunks per row
  static constexpr int kCPL = kCPR / G;        // chunks per lane
  static constexpr int kWPL = kCPL * 4;        // 32-bit words per lane
  static constexpr int kDL = D / G;            // elements per lane
  static_assert(kCPR % G == 0 && kCPL >= 1, "row must split into whole chunks");
};

// gfx950 LDS: 64 banks of 4 bytes, i.e. 256-byte bank lines.  Rows are
// stored densely and the 16-byte chunks of each row are XOR-permuted so that
// 16 consecutive rows reading the same logical chunk (the access pattern of a
// row-shifted tile) hit 16 distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int lds_chunk(int r, int c) {
  constexpr int kRowsPerLine = CPR >= 16 ? 1 : 16 / CPR;
  constexpr int kMask = (CPR >= 16 ? 16 : CPR) - 1;
  return c ^ ((r / kRowsPerLine) & kMask);
}

// ---------------------------------------------------------------------------
// Fragment loads and stores.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__device__ __forceinline__ void frag_load_global(const char* row, int part,
                                                 uint32_t (&f)[Geom<T, D, G>::kWPL]) {
  using Gm = Geom<T, D, G>;
  const u32x4* p = reinterpret_cast<const u32x4*>(row) + part;
#pragma unroll
  for (int t = 0; t < Gm::kCPL; ++t) {
    const u32x4 x = __builtin_nontemporal_load(p + t * G);
    f[4 * t + 0] = x.x;
    f[4 * t + 1] = x.y;
    f[4 * t + 2] = x.z;
    f[4 * t + 3] = x.w;
  }
}

// Same as above through the regular cache path (for rows that are re-read).
template <typename T, int D, int G>
__device__ __forceinline__ void frag_load_cached(const char* row, int part,
                                                 uint32_t (&f)[Geom<T, D, G>::kWPL]) {
  using Gm = Geom<T, D, G>;
  const u32x4* p = reinterpret_cast<const u32x4*>(row) + part;
#pragma unroll
  for (int t = 0; t < Gm::kCPL; ++t) {
    const u32x4 x = p[t * G];
    f[4 * t + 0] = x.x;
    f[4 * t + 1] = x.y;
    f[4 * t + 2] = x.z;
    f[4 * t + 3] = x.w;
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void frag_load_lds(const char* base, int r, int part,
                                              uint32_t (&f)[Geom<T, D, G>::kWPL]) {
  using Gm = Geom<T, D, G>;
  const char* row = base + r * Gm::kRowBytes;
#pragma unroll
  for (int t = 0; t < Gm::kCPL; ++t) {
    const int c = lds_chunk<Gm::kCPR>(r, t * G + part);
    const u32x4 x = *reinterpret_cast<const u32x4*>(row + c * 16);
    f[4 * t + 0] = x.x;
    f[4 * t + 1] = x.y;
    f[4 * t + 2] = x.z;
    f[4 * t + 3] = x.w;
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void frag_store_lds(char* base, int r, int part,
                                               const uint32_t (&f)[Geom<T, D, G>::kWPL]) {
  using Gm = Geom<T, D, G>;
  char* row = base + r * Gm::kRowBytes;
#pragma unroll
  for (int t = 0; t < Gm::kCPL; ++t) {
    const int c = lds_chunk<Gm::kCPR>(r, t * G + part);
    *reinterpret_cast<u32x4*>(row + c * 16) = u32x4{f[4 * t + 0], f[4 * t + 1], f[4 * t + 2], f[4 * t + 3]};
  }
}

// Copy `rows` rows of D elements of two tensors (a and b, rows `rs_a` and
// `rs_b` bytes apart in global memory) into LDS in the swizzled layout.
// Consecutive threads move consecutive 16-byte chunks, so the global reads
// are coalesced within each row.  Each thread requests up to kStageBatch
// chunks of both tensors before it writes any of them: one load followed by
// its LDS write per step would wait out a full memory round trip per chunk.
// kLastUse marks the final read of the data: those loads are issued
// non-temporal so they do not displace lines that will be read again.
constexpr int kStageBatch = 4;

template <typename T, int D, int NT, bool kLastUse>
__device__ __forceinline__ void stage2_rows_lds(char* lds_a, const char* src_a, size_t rs_a,
                                                char* lds_b, const char* src_b, size_t rs_b,
                                                int rows, int tid) {
  using Gm = Geom<T, D, 1>;
  const int total = rows * Gm::kCPR;
  for (int base = tid; base < total; base += kStageBatch * NT) {
    u32x4 xa[kStageBatch], xb[kStageBatch];
#pragma unroll
    for (int i = 0; i < kStageBatch; ++i) {
      const int idx = base + i * NT;
      if (idx < total) {
        const int r = idx / Gm::kCPR;
        const int c = idx % Gm::kCPR;
        const u32x4* sa = reinterpret_cast<const u32x4*>(src_a + r * rs_a) + c;
        const u32x4* sb = reinterpret_cast<const u32x4*>(src_b + r * rs_b) + c;
        if constexpr (kLastUse) {
          xa[i] = __builtin_nontemporal_load(sa);
          xb[i] = __builtin_nontemporal_load(sb);
        } else {
          xa[i] = *sa;
          xb[i] = *sb;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kStageBatch; ++i) {
      const int idx = base + i * NT;
      if (idx < total) {
        const int r = idx / Gm::kCPR;
        const int c = idx % Gm::kCPR;
        const int off = r * Gm::kRowBytes + lds_chunk<Gm::kCPR>(r, c) * 16;
        *reinterpret_cast<u32x4*>(lds_a + off) = xa[i];
        *reinterpret_cast<u32x4*>(lds_b + off) = xb[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Arithmetic on fragments (fp32 accumulation for both element types).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T, int WPL>
struct FragMath;

template <int WPL>
struct FragMath<float, WPL> {
  static constexpr int kDL = WPL;
  __device__ static __forceinline__ float dot(const uint32_t (&a)[WPL], const uint32_t (&b)[WPL]) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < WPL; ++t)
      s[t & 3] = __builtin_fmaf(__uint_as_float(a[t]), __uint_as_float(b[t]), s[t & 3]);
    return (s[0] + s[1]) + (s[2] + s[3]);
  }
  __device__ static __forceinline__ void axpy(float (&acc)[kDL], float p, const uint32_t (&v)[WPL]) {
#pragma unroll
    for (int t = 0; t < WPL; ++t) acc[t] = __builtin_fmaf(p, __uint_as_float(v[t]), acc[t]);
  }
  // x += c1 * v and y += c2 * v with one read of v.
  __device__ static __forceinline__ void axpy2(float (&x)[kDL], float c1, float (&y)[kDL], float c2,
                                               const uint32_t (&v)[WPL]) {
#pragma unroll
    for (int t = 0; t < WPL; ++t) {
      const float e = __uint_as_float(v[t]);
      x[t] = __builtin_fmaf(c1, e, x[t]);
      y[t] = __builtin_fmaf(c2, e, y[t]);
    }
  }
};

template <int WPL>
struct FragMath<bf16_t, WPL> {
  static constexpr int kDL = 2 * WPL;
  __device__ static __forceinline__ float dot(const uint32_t (&a)[WPL], const uint32_t (&b)[WPL]) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < WPL; ++t)
      s[t & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[t]),
                                                 __builtin_bit_cast(bf16x2_t, b[t]), s[t & 3],
                                                 false);
    return (s[0] + s[1]) + (s[2] + s[3]);
  }
  __device__ static __forceinline__ void axpy(float (&acc)[kDL], float p, const uint32_t (&v)[WPL]) {
#pragma unroll
    for (int t = 0; t < WPL; ++t) {
      acc[2 * t + 0] = __builtin_fmaf(p, bf16_lo(v[t]), acc[2 * t + 0]);
      acc[2 * t + 1] = __builtin_fmaf(p, bf16_hi(v[t]), acc[2 * t + 1]);
    }
  }
  __device__ static __forceinline__ void axpy2(float (&x)[kDL], float c1, float (&y)[kDL], float c2,
                                               const uint32_t (&v)[WPL]) {
#pragma unroll
    for (int t = 0; t < WPL; ++t) {
      const float lo = bf16_lo(v[t]);
      const float hi = bf16_hi(v[t]);
      x[2 * t + 0] = __builtin_fmaf(c1, lo, x[2 * t + 0]);
      x[2 * t + 1] = __builtin_fmaf(c1, hi, x[2 * t + 1]);
      y[2 * t + 0] = __builtin_fmaf(c2, lo, y[2 * t + 0]);
      y[2 * t + 1] = __builtin_fmaf(c2, hi, y[2 * t + 1]);
    }
  }
};

// Sum over the G lanes of a group (all lanes of the group must be active).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  if constexpr (G >= 8) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  }
  if constexpr (G >= 4) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  }
  if constexpr (G >= 2) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  }
  return x;
}

// Two fp32 values rounded to bf16 (nearest even) and packed, x in the low
// half: one v_cvt_pk_bf16_f32 (two scalar conversions would take four
// instructions with the shift and the or).
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_cvt){x, y}, bf16x2_cvt));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Signed key displacements of head h, built in LDS by thread 0 from the
// head's (a, b, lim) or its slice of the distance table: -f and +f for every
// distance f > 0, and 0 once when it is a distance.  `dist` is LDS scratch of
// kMaxOffsets ints.  Callers synchronise before reading `deltas` / `count`.
template <int MH>
__device__ __forceinline__ void build_deltas(const HeadTableT<MH>& ht, int h, int* dist,
                                             int* deltas, int* count) {
  int n;
  if (ht.table) {
    n = ht.b[h];
    for (int i = 0; i < n; ++i) dist[i] = ht.table[ht.a[h] + i];
  } else {
    n = fib_offsets_gen(ht.a[h], ht.b[h], ht.lim[h], dist, kMaxOffsets);
  }
  const int m = n < kMaxOffsets ? n : kMaxOffsets;
  int c = 0;
  for (int i = 0; i < m; ++i) {
    const int f = dist[i];
    if (f == 0) {
      deltas[c++] = 0;
    } else {
      deltas[c++] = -f;
      deltas[c++] = f;
    }
  }
  *count = c;
}

// Whether `delta` is one of the head's `count` signed displacements.
__device__ __forceinline__ bool has_delta(const int* deltas, int count, int delta) {
  bool found = false;
  for (int i = 0; i < count; ++i) found |= deltas[i] == delta;
  return found;
}

}  // namespace fibatt
