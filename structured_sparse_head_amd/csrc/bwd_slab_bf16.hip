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
// Per slab, with K and V (bf16) in LDS:
//  1. Query pass (two lanes per query row, see slab_bf16_common.h): for every
//     signed displacement, P and dP from two dot products, kept in an LDS
//     table indexed by (row, displacement); D exactly as sum P dP in fp32.
//  2. dQ pass: dS = P (dP - D) and dQ = sum dS K, re-reading K; the table
//     entries become (P, dS / sqrt(d)).
//  3. Q and dO of every row replace K and V in LDS, widened to fp32.
//  4. Key passes: the support is symmetric in j and k, so key k is seen by
//     the queries k - delta for the same displacements; dV gathers P dO_j
//     and then dK gathers dS Q_j from the table and the fp32 rows.  Every output row
//     has one writer: no atomics, bitwise reproducible.
// Q, K, V, dO and LSE are each read from HBM once; dQ, dK, dV written once.
#include "slab_bf16_common.h"

namespace fibatt {
namespace {

using namespace slab;

constexpr int kTableCols = 2 * kMaxPos + 1;  // +f (0..11), -f (12..23), 0 (24)

// LDS: per sequence row, bf16 K and V plus an fp32 copy of K for the query
// and dQ passes, later overlaid by fp32 Q and dO rows for the key passes;
// then the (P, dS) table with one row per lane pair (kMaxRows), so lanes past
// the last sequence row own private rows.
constexpr int kLdsPerRow = 2 * kBf16Stride + kF32Stride;  // >= 2 * kF32Stride
constexpr int kTableBytes = kMaxRows * kTableCols * 8;
constexpr int kLdsMax = 160 * 1024;
constexpr int kMaxRowsBwd = (kLdsMax - kTableBytes) / kLdsPerRow;  // 201

template <int MH>
struct Args {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  int H;
  int N;
  int slabs;
  float c;      // log2(e) / sqrt(64)
  float scale;  // 1 / sqrt(64)
  u32x4 rec[MH];
};

struct Prefetch {
  u32x4 k[kChunksPerThread];
  u32x4 v[kChunksPerThread];
  u32x4 q[4];
  u32x4 dout[4];
  float lse;
};

// Loads are unconditional (indices clamped into the slab) so every prefetch
// register is overwritten each time; only the LDS commit is masked.
// With `idle` set (no next slab) every address collapses onto the slab's
// first row, so the loads still retire in order but cost no HBM traffic.
template <typename A>
__device__ __forceinline__ void issue_prefetch(const A& a, int N, size_t slab, int tid, int row,
                                               int part, bool idle, Prefetch& pf) {
  const size_t base = slab * static_cast<size_t>(N) * kRowBytes;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k + base);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v + base);
  const int last = idle ? 0 : N * (kRowBytes / 16) - 1;
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    int idx = tid + c * kThreads;
    idx = idx < last ? idx : last;
    pf.k[c] = __builtin_nontemporal_load(ks + idx);
    pf.v[c] = __builtin_nontemporal_load(vs + idx);
  }
  const int r = idle ? 0 : (row < N ? row : N - 1);
  const size_t off = base + static_cast<size_t>(r) * kRowBytes + part * 64;
  const u32x4* qs = reinterpret_cast<const u32x4*>(a.q + off);
  const u32x4* ds = reinterpret_cast<const u32x4*>(a.dout + off);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    pf.q[t] = __builtin_nontemporal_load(qs + t);
    pf.dout[t] = __builtin_nontemporal_load(ds + t);
  }
  pf.lse = __builtin_nontemporal_load(a.lse + slab * static_cast<size_t>(N) + r);
}

// Makes the compiler wait here for every prefetch register.
__device__ __forceinline__ void settle(const Prefetch& pf) {
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) asm volatile("" ::"v"(pf.k[c]), "v"(pf.v[c]));
#pragma unroll
  for (int t = 0; t < 4; ++t) asm volatile("" ::"v"(pf.q[t]), "v"(pf.dout[t]));
  asm volatile("" ::"v"(pf.lse));
}

__device__ __forceinline__ void commit_kv(char* lds_k, char* lds_v, char* lds_kf, int N, int tid,
                                          const Prefetch& pf) {
  const int chunks = N * (kRowBytes / 16);
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    const int idx = tid + c * kThreads;
    if (idx < chunks) {
      const int off = (idx >> 3) * kBf16Stride + (idx & 7) * 16;
      *reinterpret_cast<u32x4*>(lds_k + off) = pf.k[c];
      *reinterpret_cast<u32x4*>(lds_v + off) = pf.v[c];
      const u32x4 x = pf.k[c];
      char* kf = lds_kf + (idx >> 3) * kF32Stride + (idx & 7) * 32;
      *reinterpret_cast<u32x4*>(kf) = u32x4{x.x << 16, x.x & 0xffff0000u, x.y << 16, x.y & 0xffff0000u};
      *reinterpret_cast<u32x4*>(kf + 16) =
          u32x4{x.z << 16, x.z & 0xffff0000u, x.w << 16, x.w & 0xffff0000u};
    }
  }
}

// A finished fp32 half-row waiting to be written: its eight 16-byte chunks
// are stored one per step of a later pass instead of in one burst, so the
// stores of all waves trickle out while they compute.
struct Pending {
  float4* dst;
  const float (&x)[32];
  float scale;
  int next;
  __device__ __forceinline__ void store(int t) {
    switch (t) {
#define FIBATT_CHUNK(T)                                                                      \
  case T:                                                                                    \
    dst[T] = make_float4(x[4 * T] * scale, x[4 * T + 1] * scale, x[4 * T + 2] * scale,        \
                         x[4 * T + 3] * scale);                                             \
    break;
      FIBATT_CHUNK(0) FIBATT_CHUNK(1) FIBATT_CHUNK(2) FIBATT_CHUNK(3)
      FIBATT_CHUNK(4) FIBATT_CHUNK(5) FIBATT_CHUNK(6) FIBATT_CHUNK(7)
#undef FIBATT_CHUNK
      default:
        break;
    }
  }
  __device__ __forceinline__ void tick() {
    if (next < 8) store(next);
    ++next;
  }
  __device__ __forceinline__ void flush() {
    for (; next < 8; ++next) store(next);
  }
};

struct NoTick {
  __device__ __forceinline__ void tick() {}
};

// Ascending positive distances of a head, one byte each in three words
// (wave-uniform, so extraction is scalar arithmetic).
struct Dist {
  uint32_t w0, w1, w2;
  __device__ __forceinline__ int at(int i) const {
    const uint32_t w = i < 4 ? w0 : (i < 8 ? w1 : w2);
    return static_cast<int>((w >> (8 * (i & 3))) & 0xffu);
  }
};

// Query pass for displacements SGN * f_i, i < n (wave-uniform n) of data row
// `row`: P (0 where the key is out of range) and dP go to table row trow,
// column base + i (written by the pair's first lane, wr), and sum P dP is
// added to d.  Two steps per
// trip, so one step's K and V fragments are in flight during the other's
// arithmetic.
template <int SGN>
__device__ __forceinline__ void query_pass(const char* lds_k, const char* lds_v, float2* tbl,
                                           Dist dist, int n, int row, int trow, int N, int part,
                                           const uint32_t (&qw)[16], const uint32_t (&dw)[16],
                                           float c, float lse2, int base, bool wr, float& d) {
  u32x4 ka[4], va[4], kb[4], vb[4];
  auto load = [&](int i, u32x4 (&kf)[4], u32x4 (&vf)[4]) {
    const int r = clamp_row(row + SGN * dist.at(i), N);
    load_bf16_half(lds_k, r, part, kf);
    load_bf16_half(lds_v, r, part, vf);
  };
  auto step = [&](int i, const u32x4 (&kf)[4], const u32x4 (&vf)[4]) {
    const int kk = row + SGN * dist.at(i);
    const float s = dot_bf16(qw, kf);
    const float dp = dot_bf16(dw, vf);
    const bool ok = static_cast<unsigned>(kk) < static_cast<unsigned>(N);
    const float p = ok ? fast_exp2(__builtin_fmaf(s, c, -lse2)) : 0.f;
    if (wr) tbl[trow * kTableCols + base + i] = make_float2(p, dp);
    d = __builtin_fmaf(p, dp, d);
  };
  if (n > 0) load(0, ka, va);
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) load(i + 1, kb, vb);
    step(i, ka, va);
    if (i + 1 < n) {
      if (i + 2 < n) load(i + 2, ka, va);
      step(i + 1, kb, vb);
    }
  }
}

// dQ pass: dS = P (dP - D) from the row's table entries, acc += dS K; the
// entry becomes (P, dS / sqrt(d)) for the key pass.
template <int SGN>
__device__ __forceinline__ void dq_pass(const char* lds_kf, float2* tbl, Dist dist, int n, int row,
                                        int trow, int N, int part, float d, float scale, int base,
                                        bool wr, float (&acc)[32]) {
  // The step's table entry is fetched with its fp32 K fragment, one step
  // ahead.
  u32x4 ka[8], kb[8];
  float2 ea, eb;
  float2* e0 = tbl + trow * kTableCols + base;
  auto load = [&](int i, u32x4 (&kf)[8], float2& e) {
    load_f32_half(lds_kf, clamp_row(row + SGN * dist.at(i), N), part, kf);
    e = e0[i];
  };
  auto step = [&](int i, const u32x4 (&kf)[8], const float2& e) {
    const float ds = e.x * (e.y - d);
    axpy_f32(acc, ds, kf);
    if (wr) e0[i] = make_float2(e.x, ds * scale);
  };
  if (n > 0) load(0, ka, ea);
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) load(i + 1, kb, eb);
    step(i, ka, ea);
    if (i + 1 < n) {
      if (i + 2 < n) load(i + 2, ka, ea);
      step(i + 1, kb, eb);
    }
  }
}

// Key pass for key row k over displacements SGN * f_i: the queries
// j = k - SGN * f_i contribute w_j * X_j, where w_j is component C of their
// table entry (P for dV, dS / sqrt(d) for dK) and X_j their fp32 row.
template <int SGN, int C, typename Tick>
__device__ __forceinline__ void key_pass(const char* lds_x, const float2* tbl, Dist dist, int n,
                                         int k, int N, int part, int base, float (&acc)[32],
                                         Tick& tk) {
  // Row and weight of a step are fetched together, one step ahead.
  u32x4 xa[8], xb[8];
  float wa, wb;
  auto load = [&](int i, u32x4 (&xf)[8], float& w) {
    const int j = k - SGN * dist.at(i);
    const int jc = clamp_row(j, N);
    load_f32_half(lds_x, jc, part, xf);
    const float2 t = tbl[jc * kTableCols + base + i];
    const bool ok = static_cast<unsigned>(j) < static_cast<unsigned>(N);
    w = ok ? (C == 0 ? t.x : t.y) : 0.f;
  };
  auto step = [&](const u32x4 (&xf)[8], float w) {
    tk.tick();
    axpy_f32(acc, w, xf);
  };
  if (n > 0) load(0, xa, wa);
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) load(i + 1, xb, wb);
    step(xa, wa);
    if (i + 1 < n) {
      if (i + 2 < n) load(i + 2, xa, wa);
      step(xb, wb);
    }
  }
}

template <int MH>
__global__ void __launch_bounds__(kThreads) bwd_slab_bf16_kernel(Args<MH> a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int row0 = 32 * wave + (lane & 31);
  const int part0 = lane >> 5;
  const int r0 = 32 * wave;

  // The grid never exceeds the slab count.  The first slab's loads are
  // completed before the loop so that the loop's first trip and later trips
  // see the same pending memory operations (the later ones wait only for
  // loads, never for the stores issued after them).
  Prefetch pf;
  int slab = blockIdx.x;
  issue_prefetch(a, a.N, slab, tid, row0, part0, false, pf);
  settle(pf);
  for (; slab < a.slabs; slab += gridDim.x) {
    // An opaque per-slab copy of N keeps row-address arithmetic inside the
    // loop instead of hoisted into registers for its whole duration.
    int N = a.N;
    asm volatile("" : "+s"(N));
    int row = row0, part = part0;  // likewise for per-lane offsets
    asm volatile("" : "+v"(row), "+v"(part));
    __syncthreads();  // the previous slab is no longer read from LDS
    // Passes 1-2: K, V in bf16.  Passes 3-4: Q, dO in fp32 over the same
    // bytes.  Then the (P, dS) table, row-major with kTableCols entries.
    char* lds_k = smem;
    char* lds_v = smem + N * kBf16Stride;
    char* lds_kf = smem + 2 * N * kBf16Stride;
    char* lds_q = smem;
    char* lds_do = smem + N * kF32Stride;
    float2* tbl = reinterpret_cast<float2*>(smem + N * kLdsPerRow);
    // Lanes past the last row repeat row N - 1 exactly (their extra terms
    // are exact zeros; their table rows are private), so every lane and wave
    // runs the same code and stores without branches: the memory wait
    // counter then tracks stores exactly and never has to drain them early.
    const bool mine = row < N;
    const int rr = mine ? row : N - 1;
    const int w0 = r0 < N ? r0 : N - 1;                 // this wave's rows: [w0, wl]
    const int wl = (r0 + 31 < N ? r0 + 31 : N - 1);
    commit_kv(lds_k, lds_v, lds_kf, N, tid, pf);
    uint32_t qw[16], dw[16];
    unpack_words(pf.q, qw);
    unpack_words(pf.dout, dw);
    const float lse2 = pf.lse * kLog2e;
    __syncthreads();
    // Start the next slab's loads; they land while this slab is computed.
    // The wait counter retires memory operations in issue order, and every
    // store of this slab is issued after these loads, so the commit at the
    // next slab never waits for those stores.
    const int next = slab + gridDim.x;
    issue_prefetch(a, N, next < a.slabs ? next : slab, tid, row, part, next >= a.slabs, pf);
    const size_t grow = static_cast<size_t>(slab) * N + rr;
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
    const bool wr = part == 0;  // table rows: row (private per lane pair)
    float dqa[32];
    {
      float d = 0.f;
      query_pass<+1>(lds_k, lds_v, tbl, dist, n_up, rr, row, N, part, qw, dw, a.c, lse2, 0, wr, d);
      query_pass<-1>(lds_k, lds_v, tbl, dist, n_dn, rr, row, N, part, qw, dw, a.c, lse2, kMaxPos,
                     wr, d);
      if (has0) {
        u32x4 kb[4], vb[4];
        load_bf16_half(lds_k, rr, part, kb);
        load_bf16_half(lds_v, rr, part, vb);
        const float s = dot_bf16(qw, kb);
        const float dp = dot_bf16(dw, vb);
        const float p = fast_exp2(__builtin_fmaf(s, a.c, -lse2));
        if (wr) tbl[row * kTableCols + z] = make_float2(p, dp);
        d = __builtin_fmaf(p, dp, d);
      }
      float (&acc)[32] = dqa;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = 0.f;
      dq_pass<+1>(lds_kf, tbl, dist, n_up, rr, row, N, part, d, a.scale, 0, wr, acc);
      dq_pass<-1>(lds_kf, tbl, dist, n_dn, rr, row, N, part, d, a.scale, kMaxPos, wr, acc);
      if (has0) {
        u32x4 kb[4];
        load_bf16_half(lds_k, rr, part, kb);
        const float2 e = tbl[row * kTableCols + z];
        const float ds = e.x * (e.y - d);
        axpy_bf16(acc, ds, kb);
        if (wr) tbl[row * kTableCols + z] = make_float2(e.x, ds * a.scale);
      }
    }
    // The next slab's loads (issued a whole pass ago) complete here, before
    // any store of this slab: the wait counter retires memory operations in
    // issue order, so no later wait has to drain this slab's stores.
    settle(pf);
    __syncthreads();  // K and V are no longer read; the table is complete
    if (mine) {
      store_f32_half_from_bf16(lds_q, row, part, qw);
      store_f32_half_from_bf16(lds_do, row, part, dw);
    }
    __syncthreads();
    {
      // Key k, displacement +f: query k - f exists while k >= f (f <= wl for
      // some key of the wave); displacement -f: query k + f < N.
      // dQ is written during the dV pass and dV during the dK pass.
      Pending pq{reinterpret_cast<float4*>(a.dq + grow * 64) + part * 8, dqa, a.scale, 0};
      float acc[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = 0.f;
      key_pass<+1, 0>(lds_do, tbl, dist, n_dn, rr, N, part, 0, acc, pq);
      key_pass<-1, 0>(lds_do, tbl, dist, n_up, rr, N, part, kMaxPos, acc, pq);
      if (has0) {
        u32x4 xb[8];
        load_f32_half(lds_do, rr, part, xb);
        axpy_f32(acc, tbl[rr * kTableCols + z].x, xb);
      }
      pq.flush();
      Pending pv{reinterpret_cast<float4*>(a.dv + grow * 64) + part * 8, acc, 1.0f, 0};
      float acc2[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) acc2[e] = 0.f;
      key_pass<+1, 1>(lds_q, tbl, dist, n_dn, rr, N, part, 0, acc2, pv);
      key_pass<-1, 1>(lds_q, tbl, dist, n_up, rr, N, part, kMaxPos, acc2, pv);
      if (has0) {
        u32x4 xb[8];
        load_f32_half(lds_q, rr, part, xb);
        axpy_f32(acc2, tbl[rr * kTableCols + z].y, xb);
      }
      pv.flush();
      store_f32_half_global(a.dk + grow * 64, part, acc2, 1.0f);
    }
  }
}

template <int MH>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    hipStream_t stream) {
  Args<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.dout = static_cast<const char*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.H = p.H;
  a.N = p.N;
  a.slabs = p.B * p.H;
  a.scale = 0.125f;  // 1 / sqrt(64)
  a.c = kLog2e * 0.125f;
  if (!pack_records(p, a.rec, MH)) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(p.N) * kLdsPerRow + kTableBytes;
  auto kern = bwd_slab_bf16_kernel<MH>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
      kMaxRowsBwd * kLdsPerRow + kTableBytes);
  if (attr != hipSuccess) return attr;
  const int cus = cu_count();
  const int grid = a.slabs < cus ? a.slabs : cus;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool bwd_slab_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && p.D == 64 && p.N <= kMaxRowsBwd && records_fit(p);
}

hipError_t launch_bwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, hipStream_t stream) {
  if (p.H <= kSmallHeads) return launch_t<kSmallHeads>(p, q, k, v, lse, dout, dq, dk, dv, stream);
  return launch_t<kMaxHeads>(p, q, k, v, lse, dout, dq, dk, dv, stream);
}

}  // namespace fibatt
