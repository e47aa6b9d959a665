// Backward kernel specialised for short bf16 sequences with d_h = 64
// (ViT-scale token counts): one persistent workgroup per CU walks a strided
// list of (b, h) slabs and loads the next slab while computing the current
// one.  Gradients are the exact derivative of the forward (Fibottention
// paper, method section, eq. (1) and (3); README Algorithm 3):
//   D_j   = sum_k P_jk dP_jk,  dP_jk = dO_j . V_k,
//   dS_jk = P_jk (dP_jk - D_j),
//   dQ_j  = sum_k dS_jk K_k / sqrt(d),
//   dK_k  = sum_j dS_jk Q_j / sqrt(d),
//   dV_k  = sum_j P_jk dO_j,
// with P_jk = exp(S_jk - LSE_j) from the forward's log-sum-exp.
//
// Lanes.  1024 threads (16 waves, four per SIMD so that LDS and arithmetic
// latency is hidden by other waves); four lanes own a row: lane l of wave w
// works on row 16 b_w + (l % 16), b_w the wave's row block (plan_blocks),
// and, with p = (l / 16) xor parity((l % 16) / 4)
// (see slab_bf16_common.h), on the element groups {4 g .. 4 g + 3} for
// g = p, p + 4, p + 8, p + 12.  The four lanes of a row
// therefore cover each 64-byte span of an fp32 output row together, so every
// global store instruction writes whole 64-byte pieces.  LDS rows are kept
// permuted (each lane's 16 elements contiguous, in that group order) so a
// lane reads its fragment with consecutive 16-byte loads.  A dot product
// ends with v_permlane32_swap and v_permlane16_swap sums.
//
// Per slab, with K and V (bf16) and an fp32 copy of K in LDS:
//  1. Query pass: for every signed displacement, P and dP from two dot
//     products, kept in an LDS table indexed by (row, displacement); D
//     exactly as sum P dP in fp32.
//  2. dQ pass: dS = P (dP - D) and dQ = sum dS K; the table entries become
//     (P, dS / sqrt(d)).
//  3. Q and dO of every row replace K and V in LDS, widened to fp32.
//  4. Key passes: the support is symmetric in j and k, so key k is seen by
//     the queries k - delta for the same displacements; dV gathers P dO_j
//     and then dK gathers dS Q_j from the table and the fp32 rows.  Every
//     output row has one writer: no atomics, bitwise reproducible.
// Q, K, V, dO and LSE are each read from HBM once; dQ, dK, dV written once,
// dQ and dV a chunk per step of the following pass rather than in bursts.
//
// Class-token mask (CLS): a row j >= 1 whose distance j to token 0 is not a
// head distance pairs with token 0 in both roles.  As query j it meets key 0
// (one more term of D_j and dQ_j, with K_0 and V_0 from LDS); as key j it is
// met by query 0 (one more term of dK_j and dV_j, from Q_0 and dO_0, which
// the lanes of row 0 stage in LDS, and the dense D_0).  Row 0 and column 0
// are dense, and two of the waves without rows of their own (there are at
// least three for N <= 201) compute them from the slab in LDS: during the
// query passes one takes row 0 (D_0, dQ_0 and row 0's table entries for the
// key passes); during the key passes the other sums column 0,
// dV_0 = sum_j P_j0 dO_j and dK_0 = sum_j dS_j0 Q_j / sqrt(d), from the fp32
// Q and dO rows and each row's pair with token 0, which the rows leave in
// LDS.  The lanes of row 0 then only stage Q_0 and dO_0: their table row is
// a discard row and their dQ, dK and dV stores go to a discard row of the
// workspace.  The class-token areas live in table rows no lane uses (lanes
// own table rows below 16 ceil(N / 16) <= 208).
#include <type_traits>

#include "slab_bf16_common.h"

namespace fibatt {
namespace {

using namespace slab;

constexpr int kThreadsB = 1024;                       // 16 waves
constexpr int kRowsB = kThreadsB / 4;                 // 256 rows, four lanes each
constexpr int kChunksB = kRowsB * (kRowBytes / 16) / kThreadsB;  // 2
constexpr int kTableCols = 2 * kMaxPos + 1;  // +f (0..11), -f (12..23), 0 (24)
constexpr int kGroups = (kMaxPos + 3) / 4;   // distance groups of four in the query pass

// LDS: per sequence row, bf16 K and V plus an fp32 copy of K for the query
// and dQ passes, later overlaid by fp32 Q and dO rows for the key passes;
// then the (P, dS) table with one row per lane group (kRowsB), so lanes past
// the last sequence row own private rows.
constexpr int kLdsPerRow = 2 * kBf16Stride + kF32Stride;  // >= 2 * kF32Stride
constexpr int kTableBytes = kRowsB * kTableCols * 8;
constexpr int kLdsMax = 160 * 1024;
constexpr int kMaxRowsBwd = (kLdsMax - kTableBytes) / kLdsPerRow;  // 201
// Class-token areas, from table row kClsRow on: bf16 Q_0 and dO_0 (256
// bytes), then per row its key-role pair with query 0, (P, dP) ("side"),
// its pair with key 0 as query, (P, dS / sqrt(d)) ("colv"), D_0, and row 0's
// (P, dP) per key.  Table row kDiscardRow takes the table writes of row 0's
// own lanes.
constexpr int kClsRow = 16 * ((kMaxRowsBwd + 15) / 16);  // 208
constexpr int kClsBytes = 256 + 2 * kRowsB * 8 + 16 + kRowsB * 8;
constexpr int kDiscardRow = kRowsB - 1;
static_assert(kClsRow * kTableCols * 8 + kClsBytes <= kDiscardRow * kTableCols * 8,
              "class-token areas must fit in the unused table rows");

// With STR the rows of every tensor follow their layouts (strided views,
// e.g. of a fused QKV projection); without it they are dense [B, H, N, 64].
template <int MH, bool STR>
struct Args {
  static constexpr bool kStrided = STR;
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* discard;  // class-token mask: 64 floats that row 0's own lanes store to
  int H;
  int N;
  int slabs;
  float c;      // log2(e) / sqrt(64)
  float scale;  // 1 / sqrt(64)
  uint64_t blocks;  // row block of wave w in bits 4 w .. 4 w + 3
  Layout lq, lk, lv, ldo, ldq, ldk, ldv;
  u32x4 rec[MH];
};

// Address of row r of a slab of tensor x (layout l, ES-byte elements) for
// either kind of arguments.
template <int ES, typename T, typename A>
__device__ __forceinline__ T* slab_row(const A& a, T* x, const Layout& l, size_t slab, int N,
                                       int r) {
  size_t off;
  if constexpr (A::kStrided)
    off = l.slab_bytes(slab, a.H, ES) + static_cast<size_t>(r) * l.row_bytes(ES);
  else
    off = (slab * static_cast<size_t>(N) + r) * (64 * ES);
  using C = std::conditional_t<std::is_const<T>::value, const char, char>;
  return reinterpret_cast<T*>(reinterpret_cast<C*>(x) + off);
}

// Writes this lane's 16 bf16 elements (packed in w, groups p, p + 4, p + 8,
// p + 12) as fp32 to logical chunks 4 p .. 4 p + 3 of an LDS row.
__device__ __forceinline__ void store_f32_q_lds(char* base, int r, int part,
                                                const uint32_t (&w)[8]) {
  const int o = f32_chunk(r, 4 * part);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    *reinterpret_cast<u32x4*>(base + o + (t << 4)) =
        u32x4{w[2 * t] << 16, w[2 * t] & 0xffff0000u, w[2 * t + 1] << 16,
              w[2 * t + 1] & 0xffff0000u};
}

// A lane's 16 elements of its Q (and dO) row are the 4-element groups
// part, part + 4, part + 8 and part + 12 (8 bytes each, 32 bytes apart).  The
// lanes of parts 2u and 2u + 1 (lanes l and l ^ 16) need, together, the
// 16-byte chunks u, u + 2, u + 4 and u + 6 of the row: the even part loads
// chunks u and u + 4, the odd one u + 2 and u + 6, so that each load
// instruction reads 64 contiguous bytes of every row (half the memory
// requests of 8-byte pieces), and the two exchange the halves the other
// needs (rows_of_chunks).
struct Prefetch {
  u32x4 k[kChunksB];
  u32x4 v[kChunksB];
  u32x4 qa, qb;  // chunks c0 and c0 + 4 of the Q row, c0 = part / 2 + 2 (part % 2)
  u32x4 da, db;  // the same chunks of the dO row
  float lse;
};

// This lane's groups part + 4 m (m = 0..3) as 8 words (group m in words
// 2 m, 2 m + 1) from its chunks a, b and its partner's (lane ^ 16).
__device__ __forceinline__ void rows_of_chunks(const u32x4& a, const u32x4& b, int part,
                                               uint32_t (&w)[8]) {
  const bool odd = (part & 1) != 0;
  // The even part sends the high halves of its chunks (groups 2u + 1 and
  // 2u + 9), the odd part the low halves (groups 2u + 4 and 2u + 12).
  const uint32_t o0 = odd ? a.x : a.z, o1 = odd ? a.y : a.w;
  const uint32_t o2 = odd ? b.x : b.z, o3 = odd ? b.y : b.w;
  const uint32_t i0 = __shfl_xor(o0, 16, 64), i1 = __shfl_xor(o1, 16, 64);
  const uint32_t i2 = __shfl_xor(o2, 16, 64), i3 = __shfl_xor(o3, 16, 64);
  w[0] = odd ? i0 : a.x;  // group part
  w[1] = odd ? i1 : a.y;
  w[2] = odd ? a.z : i0;  // group part + 4
  w[3] = odd ? a.w : i1;
  w[4] = odd ? i2 : b.x;  // group part + 8
  w[5] = odd ? i3 : b.y;
  w[6] = odd ? b.z : i2;  // group part + 12
  w[7] = odd ? b.w : i3;
}

// Loads are unconditional (indices clamped into the slab) so every prefetch
// register is overwritten each time; only the LDS commit is masked.  With
// `idle` set (no next slab) every address collapses onto the slab's first
// row, so the loads still retire in order but cost no HBM traffic.
template <typename A>
__device__ __forceinline__ void issue_prefetch(const A& a, int N, size_t slab, int tid, int row,
                                               int part, bool idle, Prefetch& pf) {
  const int last = idle ? 0 : N * (kRowBytes / 16) - 1;
  const int r = idle ? 0 : (row < N ? row : N - 1);
  const char* qr;
  const char* dr;
  if constexpr (A::kStrided) {
    const char* ks = slab_row<2>(a, a.k, a.lk, slab, N, 0);
    const char* vs = slab_row<2>(a, a.v, a.lv, slab, N, 0);
    const size_t rk = a.lk.row_bytes(2), rv = a.lv.row_bytes(2);
#pragma unroll
    for (int c = 0; c < kChunksB; ++c) {
      int idx = tid + c * kThreadsB;
      idx = idx < last ? idx : last;
      const int kr = idx >> 3, ch = idx & 7;  // row, 16-byte chunk
      pf.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + kr * rk) + ch);
      pf.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + kr * rv) + ch);
    }
    qr = slab_row<2>(a, a.q, a.lq, slab, N, r);
    dr = slab_row<2>(a, a.dout, a.ldo, slab, N, r);
  } else {
    const size_t base = slab * static_cast<size_t>(N) * kRowBytes;
    const u32x4* ks = reinterpret_cast<const u32x4*>(a.k + base);
    const u32x4* vs = reinterpret_cast<const u32x4*>(a.v + base);
#pragma unroll
    for (int c = 0; c < kChunksB; ++c) {
      int idx = tid + c * kThreadsB;
      idx = idx < last ? idx : last;
      pf.k[c] = __builtin_nontemporal_load(ks + idx);
      pf.v[c] = __builtin_nontemporal_load(vs + idx);
    }
    const size_t off = base + static_cast<size_t>(r) * kRowBytes;
    qr = a.q + off;
    dr = a.dout + off;
  }
  const int c0 = (part >> 1) + 2 * (part & 1);
  const u32x4* qs = reinterpret_cast<const u32x4*>(qr) + c0;
  const u32x4* ds = reinterpret_cast<const u32x4*>(dr) + c0;
  pf.qa = __builtin_nontemporal_load(qs);
  pf.qb = __builtin_nontemporal_load(qs + 4);
  pf.da = __builtin_nontemporal_load(ds);
  pf.db = __builtin_nontemporal_load(ds + 4);
  pf.lse = __builtin_nontemporal_load(a.lse + slab * static_cast<size_t>(N) + r);
}

// Makes the compiler wait here for every prefetch register.
__device__ __forceinline__ void settle(const Prefetch& pf) {
#pragma unroll
  for (int c = 0; c < kChunksB; ++c) asm volatile("" ::"v"(pf.k[c]), "v"(pf.v[c]));
  asm volatile("" ::"v"(pf.qa), "v"(pf.qb), "v"(pf.da), "v"(pf.db));
  asm volatile("" ::"v"(pf.lse));
}

__device__ __forceinline__ void commit_kv(char* lds_k, char* lds_v, char* lds_kf, int N, int tid,
                                          const Prefetch& pf) {
  const int chunks = N * (kRowBytes / 16);
#pragma unroll
  for (int c = 0; c < kChunksB; ++c) {
    const int idx = tid + c * kThreadsB;
    if (idx < chunks) {
      // Chunk ch of row r holds element groups 2 ch and 2 ch + 1 (4 elements
      // each).  Group g belongs to lane part g % 4, slot m = g / 4: in bf16
      // it is half m % 2 of logical chunk 2 (g % 4) + m / 2, in fp32 logical
      // chunk 4 (g % 4) + m.
      const int r = idx >> 3, ch = idx & 7;
      const int g0 = 2 * ch, g1 = 2 * ch + 1;
      const int b0 = b16_chunk(r, 2 * (g0 & 3) + (g0 >> 3)) + ((g0 >> 2) & 1) * 8;
      const int b1 = b16_chunk(r, 2 * (g1 & 3) + (g1 >> 3)) + ((g1 >> 2) & 1) * 8;
      const u32x4 xk = pf.k[c], xv = pf.v[c];
      *reinterpret_cast<uint2*>(lds_k + b0) = make_uint2(xk.x, xk.y);
      *reinterpret_cast<uint2*>(lds_k + b1) = make_uint2(xk.z, xk.w);
      *reinterpret_cast<uint2*>(lds_v + b0) = make_uint2(xv.x, xv.y);
      *reinterpret_cast<uint2*>(lds_v + b1) = make_uint2(xv.z, xv.w);
      char* f0 = lds_kf + f32_chunk(r, 4 * (g0 & 3) + (g0 >> 2));
      char* f1 = lds_kf + f32_chunk(r, 4 * (g1 & 3) + (g1 >> 2));
      *reinterpret_cast<u32x4*>(f0) =
          u32x4{xk.x << 16, xk.x & 0xffff0000u, xk.y << 16, xk.y & 0xffff0000u};
      *reinterpret_cast<u32x4*>(f1) =
          u32x4{xk.z << 16, xk.z & 0xffff0000u, xk.w << 16, xk.w & 0xffff0000u};
    }
  }
}

// A finished fp32 row fragment waiting to be written: its four 16-byte
// groups (64 bytes apart in the row) are stored a few steps apart during
// later passes instead of in one burst, so the stores of all waves trickle
// out while they compute.  Chunk indices are compile-time constants
// so that every store is one 16-byte store at a fixed offset.
struct Pending {
  float4* dst;
  const float (&x)[16];
  float scale;
  template <int T>
  __device__ __forceinline__ void store() const {
    dst[4 * T] = make_float4(x[4 * T] * scale, x[4 * T + 1] * scale, x[4 * T + 2] * scale,
                             x[4 * T + 3] * scale);
  }
};

// Query pass for displacements SGN * f_i, i < n (wave-uniform n) of data row
// `row`, four distances per group: each lane forms its partial Q.K and dO.V
// products for the group's four keys, and two transposed reductions leave
// the scores of distance 4 g + slot in the lane of that slot.  That lane
// writes P (0 where the key is out of range) and dP to table row trow,
// column base + i, and adds P dP to its partial d.  One fragment variable
// per distance, requested a step ahead: loads under a condition then merge
// with nothing, so the compiler needs no register copies at branch joins.
template <int SGN>
__device__ __forceinline__ void query_pass(const char* lds_k, const char* lds_v, float2* tbl,
                                           Dist dist, int n, int row, int trow, int N, int part,
                                           int slot, const uint32_t (&qw)[8],
                                           const uint32_t (&dw)[8], float c, float lse2, int base,
                                           float& d) {
  u32x4 kf[kMaxPos][2], vf[kMaxPos][2];
  auto load = [&](int i) {
    const int r = clamp_row(row + SGN * dist.at(i), N);
    load_bf16_q(lds_k + part * 32, r, kf[i]);
    load_bf16_q(lds_v + part * 32, r, vf[i]);
  };
  if (n > 0) load(0);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (4 * g < n) {
      float ps[4], pp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        ps[j] = 0.f;
        pp[j] = 0.f;
        if (i < n) {
          if (i + 1 < n) load(i + 1);
          ps[j] = dot_part(qw, kf[i]);
          pp[j] = dot_part(dw, vf[i]);
        }
      }
      const float sc = reduce4(ps);
      const float dp = reduce4(pp);
      const uint32_t w = g == 0 ? dist.w0 : (g == 1 ? dist.w1 : dist.w2);
      const int kk = row + SGN * static_cast<int>(__builtin_amdgcn_ubfe(w, 8 * slot, 8));
      const int i = 4 * g + slot;
      const bool ok = static_cast<unsigned>(kk) < static_cast<unsigned>(N);
      const float p = ok ? fast_exp2(__builtin_fmaf(sc, c, -lse2)) : 0.f;
      if (i < n) {
        tbl[trow * kTableCols + base + i] = make_float2(p, dp);
        d = __builtin_fmaf(p, dp, d);
      }
    }
  }
}

// dQ pass: dS = P (dP - D) from the row's table entries, acc += dS K; the
// entry becomes (P, dS / sqrt(d)) for the key pass.  With the class-token
// mask (colv set) the entry of displacement -row, whose key is token 0, is
// also copied to colv[row].
template <int SGN>
__device__ __forceinline__ void dq_pass(const char* lds_kf, float2* tbl, Dist dist, int n, int row,
                                        int trow, int N, int part, float d, float scale, int base,
                                        bool wr, float (&acc)[16], float2* colv = nullptr) {
  float2* e0 = tbl + trow * kTableCols + base;
  for (int i = 0; i < n; ++i) {
    const int f = dist.at(i);
    u32x4 kf[4];
    load_f32_q(lds_kf + part * 64, clamp_row(row + SGN * f, N), kf);
    const float2 e = e0[i];
    const float ds = e.x * (e.y - d);
    axpy_q(acc, ds, kf);
    const float2 r = make_float2(e.x, ds * scale);
    if (wr) e0[i] = r;
    if (SGN < 0 && colv && wr && f == row) colv[row] = r;
  }
}

// Key pass for key row k over displacements SGN * f_i: the queries
// j = k - SGN * f_i contribute w_j * X_j, where w_j is component C of their
// table entry (P for dV, dS / sqrt(d) for dK) and X_j their fp32 row (the
// other waves of the SIMD cover the LDS latency of each step).  With a
// pending fragment, its chunks T0 and T0 + 1 are stored after steps 0 and 4:
// the two passes of a kind spread a fragment's four stores over their steps.
template <int SGN, int C, int T0>
__device__ __forceinline__ void key_pass(const char* lds_x, const float2* tbl, Dist dist, int n,
                                         int k, int N, int part, int base, float (&acc)[16],
                                         const Pending* pend) {
  auto step = [&](int i) {
    const int j = k - SGN * dist.at(i);
    const int jc = clamp_row(j, N);
    u32x4 xf[4];
    load_f32_q(lds_x + part * 64, jc, xf);
    const float2 t = tbl[jc * kTableCols + base + i];
    const bool ok = static_cast<unsigned>(j) < static_cast<unsigned>(N);
    axpy_q(acc, ok ? (C == 0 ? t.x : t.y) : 0.f, xf);
  };
  int i = 0;
  if (pend) {
    if (0 < n) step(0);
    pend->store<T0>();
    if (1 < n) step(1);
    if (2 < n) step(2);
    if (3 < n) step(3);
    if (4 < n) step(4);
    pend->store<T0 + 1>();
    i = 5;
  }
  for (; i < n; ++i) step(i);
}

// Column 0 of the class-token mask for one slab, by one wave in the key
// passes: slot l % 16 of the lane takes queries slot, slot + 16, ... (N <=
// 208: at most 13 each) with the lane parts of a row block; each query's
// (P_j0, dS_j0 / sqrt(d)) is in colv, left there by its row.  A lane's sums
// are completed over the 16 lanes that hold the same part (lane l ^ x, x in
// the span of 1, 2, 12 and 20), and the lanes of slot 0 store the row, and
// copy dQ_0 into place.
constexpr int kColSlots = kClsRow / 16;  // 13

__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

template <typename A>
__device__ __forceinline__ void dense_col0(const A& a, int slab, int N, int lane, char* smem) {
  const char* lds_q = smem;
  const char* lds_do = smem + N * kF32Stride;
  const float2* tbl = reinterpret_cast<const float2*>(smem + N * kLdsPerRow);
  const float2* colv =
      reinterpret_cast<const float2*>(reinterpret_cast<const char*>(tbl + kClsRow * kTableCols) +
                                      256) + kRowsB;
  const int slot = lane & 15;
  const int part = lane_part(lane);
  // One output row at a time (dV_0 from dO, then dK_0 from Q), to keep
  // registers for the prefetch of the next slab.
  auto column = [&](const char* lds_x, bool second, float* out, const Layout& l) {
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll 1
    for (int t = 0; t < kColSlots; ++t) {
      const int j = slot + 16 * t;
      const int jc = clamp_row(j, N);
      const float2 e = colv[jc];
      const float w = j < N ? (second ? e.y : e.x) : 0.f;
      u32x4 xb[4];
      load_f32_q(lds_x + part * 64, jc, xb);
      axpy_q(acc, w, xb);
    }
    constexpr int kSpan[4] = {1, 2, 12, 20};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += wave_xor(acc[e], kSpan[s]);
    if (slot == 0) {  // lanes 0, 16, 32, 48: parts 0..3 of the row
      float4* p = reinterpret_cast<float4*>(slab_row<4>(a, out, l, slab, N, 0)) + part;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        p[4 * t] = make_float4(acc[4 * t], acc[4 * t + 1], acc[4 * t + 2], acc[4 * t + 3]);
    }
  };
  column(lds_do, false, a.dv, a.ldv);
  column(lds_q, true, a.dk, a.ldk);
}

// Class-token LDS areas (see kClsRow).
struct ClsLds {
  float2* side;  // per row: (P, dP) with query 0
  float2* colv;  // per row: (P, dS / sqrt(d)) with key 0
  float* d0;     // D_0
  float2* ppd;   // per key: (P_0k, dP_0k)
  __device__ ClsLds(char* smem, int N) {
    char* base = smem + N * kLdsPerRow + kClsRow * kTableCols * 8 + 256;
    side = reinterpret_cast<float2*>(base);
    colv = side + kRowsB;
    d0 = reinterpret_cast<float*>(colv + kRowsB);
    ppd = reinterpret_cast<float2*>(d0 + 4);
  }
};

// Row 0 of the class-token mask for one slab, by one wave during the query
// passes (same slots and parts as dense_col0): D_0 = sum_k P_0k dP_0k over
// all keys, keeping each key's (P_0k, dP_0k) in LDS, then dQ_0 =
// sum_k dS_0k K_k / sqrt(d) in a second sweep; then row 0's table entries
// (P, dS / sqrt(d)) for the keys at head distances (one lane per distance:
// looking each key's distance up in the sweep cost a loop per key), the
// diagonal and colv[0], and finally D_0 for the key passes.
template <typename A>
__device__ __forceinline__ void dense_row0(const A& a, int slab, int N, int lane, char* smem) {
  const char* lds_k = smem;
  const char* lds_v = smem + N * kBf16Stride;
  const char* lds_kf = smem + 2 * N * kBf16Stride;
  float2* tbl = reinterpret_cast<float2*>(smem + N * kLdsPerRow);
  const char* lds_r0 = reinterpret_cast<const char*>(tbl + kClsRow * kTableCols);
  const ClsLds cl(smem, N);
  const u32x4 rec = a.rec[slab % a.H];
  const Dist dist{rec.x, rec.y, rec.z};
  const int npos = static_cast<int>(rec.w & 0xffu);
  const bool has0 = ((rec.w >> 8) & 0xffu) != 0;
  const int slot = lane & 15;
  const int part = lane_part(lane);
  uint32_t q0w[8], d0w[8];
  {
    const u32x4 q0 = *reinterpret_cast<const u32x4*>(lds_r0 + part * 32);
    const u32x4 q1 = *reinterpret_cast<const u32x4*>(lds_r0 + part * 32 + 16);
    const u32x4 o0 = *reinterpret_cast<const u32x4*>(lds_r0 + 128 + part * 32);
    const u32x4 o1 = *reinterpret_cast<const u32x4*>(lds_r0 + 144 + part * 32);
    q0w[0] = q0.x; q0w[1] = q0.y; q0w[2] = q0.z; q0w[3] = q0.w;
    q0w[4] = q1.x; q0w[5] = q1.y; q0w[6] = q1.z; q0w[7] = q1.w;
    d0w[0] = o0.x; d0w[1] = o0.y; d0w[2] = o0.z; d0w[3] = o0.w;
    d0w[4] = o1.x; d0w[5] = o1.y; d0w[6] = o1.z; d0w[7] = o1.w;
  }
  const float lse2 = a.lse[static_cast<size_t>(slab) * N] * kLog2e;
  float d0 = 0.f;
#pragma unroll 1
  for (int t = 0; t < kColSlots; ++t) {
    const int k = slot + 16 * t;
    const int kc = clamp_row(k, N);
    u32x4 kb[2], vb[2];
    load_bf16_q(lds_k + part * 32, kc, kb);
    load_bf16_q(lds_v + part * 32, kc, vb);
    const float s = dot_q(q0w, kb);
    const float dp = dot_q(d0w, vb);
    const float p = k < N ? fast_exp2(__builtin_fmaf(s, a.c, -lse2)) : 0.f;
    d0 = __builtin_fmaf(p, dp, d0);
    if (part == 0) cl.ppd[k] = make_float2(p, dp);  // read back by this wave only
  }
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) d0 += wave_xor(d0, x);
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll 1
  for (int t = 0; t < kColSlots; ++t) {
    const int k = slot + 16 * t;
    const float2 pp = cl.ppd[k];
    const float ds = pp.x * (pp.y - d0);
    u32x4 kf[4];
    load_f32_q(lds_kf + part * 64, clamp_row(k, N), kf);
    axpy_q(acc, ds, kf);
  }
  // Row 0's table entries (P, dS / sqrt(d)): lane i takes head distance i
  // (query 0, displacement +f_i: table row 0, column i); lane 12 the
  // diagonal and colv[0].  The same values the sweep above used.
  if (lane < npos) {
    const int k = dist.at(lane);
    const float2 pp = cl.ppd[k];
    tbl[lane] = make_float2(pp.x, pp.x * (pp.y - d0) * a.scale);
  } else if (lane == kMaxPos) {
    const float2 pp = cl.ppd[0];
    const float2 e = make_float2(pp.x, pp.x * (pp.y - d0) * a.scale);
    cl.colv[0] = e;
    if (has0) tbl[2 * kMaxPos] = e;
  }
  constexpr int kSpan[4] = {1, 2, 12, 20};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += wave_xor(acc[e], kSpan[s]);
  if (lane == 0) *cl.d0 = d0;
  if (slot == 0) {  // lanes 0, 16, 32, 48: parts 0..3 of the row
    float4* pq = reinterpret_cast<float4*>(slab_row<4>(a, a.dq, a.ldq, slab, N, 0)) + part;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pq[4 * t] = make_float4(acc[4 * t] * a.scale, acc[4 * t + 1] * a.scale,
                              acc[4 * t + 2] * a.scale, acc[4 * t + 3] * a.scale);
  }
}

template <int MH, bool CLS, bool STR>
__global__ void __launch_bounds__(kThreadsB) bwd_slab_bf16_kernel(Args<MH, STR> a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int r0 = 16 * static_cast<int>((a.blocks >> (4 * wave)) & 15u);
  const int row0 = r0 + (lane & 15);
  const int part0 = lane_part(lane);
  const int slot0 = quad_slot(lane);

  // The grid never exceeds the slab count.  The first slab's loads are
  // completed before the loop so that the loop's first trip and later trips
  // see the same pending memory operations (the later ones wait only for
  // loads, never for the stores issued after them).
  Prefetch pf;
  int slab = blockIdx.x;
  issue_prefetch(a, a.N, slab, tid, row0, part0, false, pf);
  settle(pf);
  // Waves whose rows all lie past the sequence only help stage the slabs;
  // they run a loop of their own with the same barriers.
  if (r0 >= a.N) {
    // With the class-token mask the first wave without rows sums column 0
    // and the second one computes row 0.
    const bool colw = CLS && r0 == 16 * ((a.N + 15) / 16);
    const bool roww = CLS && r0 == 16 * ((a.N + 15) / 16 + 1);
    for (; slab < a.slabs; slab += gridDim.x) {
      int N = a.N;
      asm volatile("" : "+s"(N));
      __syncthreads();
      commit_kv(smem, smem + N * kBf16Stride, smem + 2 * N * kBf16Stride, N, tid, pf);
      __syncthreads();
      const int next = slab + gridDim.x;
      // Row 0 runs before this wave's share of the next slab's loads, so the
      // prefetch registers are free while it runs.  Those loads are not
      // waited for here: the next slab's commit does that, and waiting now
      // (a full memory round trip after row 0) held the workgroup at the
      // next barrier.
      if (roww) dense_row0(a, slab, N, lane, smem);
      issue_prefetch(a, N, next < a.slabs ? next : slab, tid, row0, part0, next >= a.slabs, pf);
      __syncthreads();
      __syncthreads();
      if (colw) dense_col0(a, slab, N, lane, smem);
    }
    return;
  }
  for (; slab < a.slabs; slab += gridDim.x) {
    // Opaque per-slab copies of N and of the lane's row and part keep the
    // address arithmetic inside the loop instead of hoisted into registers.
    int N = a.N;
    asm volatile("" : "+s"(N));
    int row = row0, part = part0, slot = slot0;
    asm volatile("" : "+v"(row), "+v"(part), "+v"(slot));
    __syncthreads();  // the previous slab is no longer read from LDS
    char* lds_k = smem;
    char* lds_v = smem + N * kBf16Stride;
    char* lds_kf = smem + 2 * N * kBf16Stride;
    char* lds_q = smem;
    char* lds_do = smem + N * kF32Stride;
    float2* tbl = reinterpret_cast<float2*>(smem + N * kLdsPerRow);
    char* lds_r0 = reinterpret_cast<char*>(tbl + kClsRow * kTableCols);  // CLS: Q_0, dO_0
    float2* side = reinterpret_cast<float2*>(lds_r0 + 256);  // CLS: row's pair with query 0
    float2* colv = side + kRowsB;                             // CLS: row's pair with key 0
    const float* d0slot = reinterpret_cast<const float*>(colv + kRowsB);  // CLS: D_0
    // Lanes past the last row repeat row N - 1 exactly (their extra terms
    // are exact zeros; their table rows are private), so every lane and wave
    // runs the same code and stores without branches: the memory wait
    // counter then tracks stores exactly and never has to drain them early.
    const bool mine = row < N;
    const int rr = mine ? row : N - 1;
    const int w0 = r0 < N ? r0 : N - 1;  // this wave's rows: [w0, wl]
    const int wl = (r0 + 15 < N ? r0 + 15 : N - 1);
    commit_kv(lds_k, lds_v, lds_kf, N, tid, pf);
    uint32_t qw[8], dw[8];
    rows_of_chunks(pf.qa, pf.qb, part, qw);
    rows_of_chunks(pf.da, pf.db, part, dw);
    const float lse2 = pf.lse * kLog2e;
    if (CLS && row == 0) {
      *reinterpret_cast<u32x4*>(lds_r0 + part * 32) = u32x4{qw[0], qw[1], qw[2], qw[3]};
      *reinterpret_cast<u32x4*>(lds_r0 + part * 32 + 16) = u32x4{qw[4], qw[5], qw[6], qw[7]};
      *reinterpret_cast<u32x4*>(lds_r0 + 128 + part * 32) = u32x4{dw[0], dw[1], dw[2], dw[3]};
      *reinterpret_cast<u32x4*>(lds_r0 + 144 + part * 32) = u32x4{dw[4], dw[5], dw[6], dw[7]};
    }
    __syncthreads();
    // Start the next slab's loads; they land while this slab is computed.
    const int next = slab + gridDim.x;
    issue_prefetch(a, N, next < a.slabs ? next : slab, tid, row, part, next >= a.slabs, pf);
    const u32x4 rec = a.rec[slab % a.H];
    const Dist dist{rec.x, rec.y, rec.z};
    const int npos = static_cast<int>(rec.w & 0xffu);
    const bool has0 = ((rec.w >> 8) & 0xffu) != 0;
    // Displacement +f has a valid pair for some query of this wave while
    // w0 + f < N, and -f while f <= wl; both are prefixes of the ascending
    // distances.  For keys the roles swap.
    int n_up = 0, n_dn = 0;
    for (int i = 0; i < npos; ++i) {
      const int f = dist.at(i);
      n_up += (w0 + f < N) ? 1 : 0;
      n_dn += (f <= wl) ? 1 : 0;
    }
    constexpr int z = 2 * kMaxPos;  // table column of distance 0
    const bool wr = part == 0;      // table rows: row (private per lane group)
    // Class-token mask: this row's pairs with token 0 (query role: P and dP
    // against key 0, after the query passes; key role: P and dP from query
    // 0, kept in side[] until the key passes know D_0).
    const bool need0 = CLS && rr >= 1 && !dist.has(rr, npos);
    const size_t r0g = static_cast<size_t>(slab) * N;  // row 0 of the slab
    if constexpr (CLS) {
      // Key role: query 0 against this row's key, from the staged Q_0, dO_0.
      u32x4 kb[2], vb[2], qz[2], dz[2];
      qz[0] = *reinterpret_cast<const u32x4*>(lds_r0 + part * 32);
      qz[1] = *reinterpret_cast<const u32x4*>(lds_r0 + part * 32 + 16);
      dz[0] = *reinterpret_cast<const u32x4*>(lds_r0 + 128 + part * 32);
      dz[1] = *reinterpret_cast<const u32x4*>(lds_r0 + 144 + part * 32);
      const uint32_t q0w[8] = {qz[0].x, qz[0].y, qz[0].z, qz[0].w,
                               qz[1].x, qz[1].y, qz[1].z, qz[1].w};
      const uint32_t d0w[8] = {dz[0].x, dz[0].y, dz[0].z, dz[0].w,
                               dz[1].x, dz[1].y, dz[1].z, dz[1].w};
      load_bf16_q(lds_k + part * 32, rr, kb);
      load_bf16_q(lds_v + part * 32, rr, vb);
      const float s0k = dot_q(q0w, kb);
      const float dp0k = dot_q(d0w, vb);
      const float lse2_0 = a.lse[r0g] * kLog2e;
      const float pk = need0 ? fast_exp2(__builtin_fmaf(s0k, a.c, -lse2_0)) : 0.f;
      if (wr) side[row] = make_float2(pk, dp0k);  // dS needs D_0: formed in the key pass
    }
    // Row 0's own lanes write a discard table row (the row-0 wave owns row 0).
    const int trow = CLS && row == 0 ? kDiscardRow : row;
    float dqa[16];
    {
      float d = 0.f;
      query_pass<+1>(lds_k, lds_v, tbl, dist, n_up, rr, trow, N, part, slot, qw, dw, a.c, lse2, 0,
                     d);
      query_pass<-1>(lds_k, lds_v, tbl, dist, n_dn, rr, trow, N, part, slot, qw, dw, a.c, lse2,
                     kMaxPos, d);
      d = quad_sum(d);
      if (has0) {
        u32x4 kb[2], vb[2];
        load_bf16_q(lds_k + part * 32, rr, kb);
        load_bf16_q(lds_v + part * 32, rr, vb);
        const float s = dot_q(qw, kb);
        const float dp = dot_q(dw, vb);
        const float p = fast_exp2(__builtin_fmaf(s, a.c, -lse2));
        if (wr) tbl[trow * kTableCols + z] = make_float2(p, dp);
        d = __builtin_fmaf(p, dp, d);
      }
      float pq = 0.f, dpq = 0.f;
      if constexpr (CLS) {
        u32x4 kb[2], vb[2];
        load_bf16_q(lds_k + part * 32, 0, kb);
        load_bf16_q(lds_v + part * 32, 0, vb);
        const float s = dot_q(qw, kb);
        dpq = dot_q(dw, vb);
        const float p0 = fast_exp2(__builtin_fmaf(s, a.c, -lse2));
        pq = need0 ? p0 : 0.f;
        d = __builtin_fmaf(pq, dpq, d);
        // This row's pair with key 0 for the column sum (a head distance's
        // pair is copied from the table after the dQ pass instead).
        if (wr && mine && need0)
          colv[rr] = make_float2(p0, p0 * (dpq - d) * a.scale);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) dqa[e] = 0.f;
      dq_pass<+1>(lds_kf, tbl, dist, n_up, rr, trow, N, part, d, a.scale, 0, wr, dqa);
      dq_pass<-1>(lds_kf, tbl, dist, n_dn, rr, trow, N, part, d, a.scale, kMaxPos, wr, dqa,
                  CLS ? colv : nullptr);
      if (has0) {
        u32x4 kf[4];
        load_f32_q(lds_kf + part * 64, rr, kf);
        const float2 e = tbl[trow * kTableCols + z];
        const float ds = e.x * (e.y - d);
        axpy_q(dqa, ds, kf);
        if (wr) tbl[trow * kTableCols + z] = make_float2(e.x, ds * a.scale);
      }
      if constexpr (CLS) {
        u32x4 kf[4];
        load_f32_q(lds_kf + part * 64, 0, kf);
        axpy_q(dqa, pq * (dpq - d), kf);
      }
    }
    // The next slab's loads (issued a whole pass ago) complete here, before
    // any store of this slab: the wait counter retires memory operations in
    // issue order, so no later wait has to drain this slab's stores.
    settle(pf);
    __syncthreads();  // K and V are no longer read; the table is complete
    if (mine) {
      store_f32_q_lds(lds_q, row, part, qw);
      store_f32_q_lds(lds_do, row, part, dw);
    }
    __syncthreads();
    {
      // Key k, displacement +f: query k - f exists while k >= f (f <= wl for
      // some key of the wave); displacement -f: query k + f < N.
      // dQ is written during the dV pass and dV during the dK pass.
      // With the class-token mask row 0's results come from elsewhere.
      const bool drop = CLS && rr == 0;
      float* dq_row = drop ? a.discard : slab_row<4>(a, a.dq, a.ldq, slab, N, rr);
      float* dv_row = drop ? a.discard : slab_row<4>(a, a.dv, a.ldv, slab, N, rr);
      float* dk_row = drop ? a.discard : slab_row<4>(a, a.dk, a.ldk, slab, N, rr);
      const Pending pq{reinterpret_cast<float4*>(dq_row) + part, dqa, a.scale};
      float acc[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
      key_pass<+1, 0, 0>(lds_do, tbl, dist, n_dn, rr, N, part, 0, acc, &pq);
      key_pass<-1, 0, 2>(lds_do, tbl, dist, n_up, rr, N, part, kMaxPos, acc, &pq);
      if (has0) {
        u32x4 xb[4];
        load_f32_q(lds_do + part * 64, rr, xb);
        axpy_q(acc, tbl[rr * kTableCols + z].x, xb);
      }
      if constexpr (CLS) {
        u32x4 xb[4];
        load_f32_q(lds_do + part * 64, 0, xb);
        axpy_q(acc, side[rr].x, xb);
      }
      const Pending pv{reinterpret_cast<float4*>(dv_row) + part, acc, 1.0f};
      float acc2[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc2[e] = 0.f;
      key_pass<+1, 1, 0>(lds_q, tbl, dist, n_dn, rr, N, part, 0, acc2, &pv);
      key_pass<-1, 1, 2>(lds_q, tbl, dist, n_up, rr, N, part, kMaxPos, acc2, &pv);
      if (has0) {
        u32x4 xb[4];
        load_f32_q(lds_q + part * 64, rr, xb);
        axpy_q(acc2, tbl[rr * kTableCols + z].y, xb);
      }
      if constexpr (CLS) {
        u32x4 xb[4];
        load_f32_q(lds_q + part * 64, 0, xb);
        const float2 e = side[rr];
        axpy_q(acc2, e.x * (e.y - *d0slot) * a.scale, xb);
      }
      float4* dk = reinterpret_cast<float4*>(dk_row) + part;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dk[4 * t] = make_float4(acc2[4 * t], acc2[4 * t + 1], acc2[4 * t + 2], acc2[4 * t + 3]);
    }
  }
}

template <int MH, bool CLS, bool STR>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    float* discard, hipStream_t stream) {
  Args<MH, STR> a;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.ldo = p.ldo;
  a.ldq = p.ldq;
  a.ldk = p.ldk;
  a.ldv = p.ldv;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.dout = static_cast<const char*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.discard = discard;
  a.H = p.H;
  a.N = p.N;
  a.slabs = p.B * p.H;
  a.scale = 0.125f;  // 1 / sqrt(64)
  a.c = kLog2e * 0.125f;
  if (!pack_records(p, a.rec, MH)) return hipErrorInvalidValue;
  a.blocks = plan_blocks(p.N, p.H, a.rec);
  const size_t lds = static_cast<size_t>(p.N) * kLdsPerRow + kTableBytes;
  auto kern = bwd_slab_bf16_kernel<MH, CLS, STR>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      kMaxRowsBwd * kLdsPerRow + kTableBytes);
  if (attr != hipSuccess) return attr;
  const int cus = cu_count();
  const int grid = a.slabs < cus ? a.slabs : cus;
  launch(kern, dim3(grid), dim3(kThreadsB), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool bwd_slab_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && p.D == 64 && p.N <= kMaxRowsBwd && records_fit(p);
}

hipError_t launch_bwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, float* discard, hipStream_t stream) {
  const bool small = p.H <= kSmallHeads;
#define FIBATT_BWD_SLAB(CLS, STR)                                                              \
  return small ? launch_t<kSmallHeads, CLS, STR>(p, q, k, v, lse, dout, dq, dk, dv, discard,   \
                                                 stream)                                       \
               : launch_t<kMaxHeads, CLS, STR>(p, q, k, v, lse, dout, dq, dk, dv, discard, stream)
  if (p.strided) {
    if (p.cls) FIBATT_BWD_SLAB(true, true);
    FIBATT_BWD_SLAB(false, true);
  }
  if (p.cls) FIBATT_BWD_SLAB(true, false);
  FIBATT_BWD_SLAB(false, false);
#undef FIBATT_BWD_SLAB
}

}  // namespace fibatt
