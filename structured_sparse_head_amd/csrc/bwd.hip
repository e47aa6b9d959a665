// Backward kernels: exact gradients of the sparse Fibottention attention.
//
// The Fibottention paper (method section, eq. (1) and (3)) and the README's
// Algorithm 3 define the forward only; the backward is its derivative.  With
// P the support-restricted softmax and dP_jk = dO_j . V_k,
//   D_j   = sum_k P_jk dP_jk,
//   dS_jk = P_jk (dP_jk - D_j),
//   dQ_j  = sum_k dS_jk K_k / sqrt(d),
//   dK_k  = sum_j dS_jk Q_j / sqrt(d),
//   dV_k  = sum_j P_jk dO_j.
// P is recomputed from the forward's log-sum-exp (P_jk = exp(S_jk - LSE_j)).
//
// D_j is summed from P and dP in fp32 rather than taken as dO_j . O_j: with
// O stored in bf16 the latter carries O's rounding into every dS of the row,
// which on peaked rows pushes dK past the bf16 error bound.  The query pass
// therefore accumulates A = sum_k P dP K and Bv = sum_k P K next to D and
// forms dQ = (A - D Bv) / sqrt(d) at the end (same sum, regrouped), so no
// second pass over the keys is needed.  O is not read.
//
// The support is symmetric in j and k (the set is defined through |j - k|),
// so the queries that see key k are exactly k + delta for the same signed
// displacements delta.  dK and dV are gathered key by key over that list:
// every output row has a single writer, no atomics, and the results are
// bitwise reproducible.
//
// Variants mirror the forward:
//  * slab: one workgroup per (b, h) slab.  K and V sit in LDS for the
//    query-centric pass (dQ and D); then Q and dO replace them for the
//    key-centric pass (dK, dV).  LSE and D of the slab stay in LDS.
//  * stream: a query launch writes dQ and D (D to the workspace); a key
//    launch then gathers dK and dV, reading shifted rows from global memory.
#include <type_traits>

#include "kernel_common.h"
#include "launch.h"

namespace fibatt {
namespace {

template <int MH>
struct BwdArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* ws;  // D per row (stream variant)
  int H;
  int N;
  int tiles;         // row tiles per slab (stream variant)
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
  Layout lq, lk, lv, ldo, ldq, ldk, ldv;
  HeadTableT<MH> ht;
};

// A slab's rows of one tensor: base pointer and byte stride.
struct Rows {
  char* base;
  size_t rs;
  __device__ char* row(int r) const { return base + static_cast<size_t>(r) * rs; }
};

template <typename T, typename P>
__device__ __forceinline__ Rows slab_rows(P* ptr, const Layout& l, size_t slab, int H) {
  constexpr int es = static_cast<int>(sizeof(T));
  return Rows{reinterpret_cast<char*>(const_cast<typename std::remove_const<P>::type*>(ptr)) +
                  l.slab_bytes(slab, H, es),
              l.row_bytes(es)};
}

template <int DL>
__device__ __forceinline__ void zero_acc(float (&acc)[DL]) {
#pragma unroll
  for (int t = 0; t < DL; ++t) acc[t] = 0.f;
}

// A lane's fragment is chunks part, part + G, part + 2 G, ... of its row
// (CH elements each: 16 bytes of the input type), so its element e sits at
// CH (G (e / CH) + part) + e % CH of the row; fp32 chunk q of the lane's
// fragment (4 elements, q = e / 4) lands at float4 index
// (CH / 4) (G (q / (CH / 4)) + part) + q % (CH / 4).
template <int CH, int G>
__device__ __forceinline__ int frag_f4(int part, int q) {
  constexpr int F = CH / 4;
  return F * (G * (q / F) + part) + q % F;
}

// Stores x * scale as fp32.
template <int DL, int CH, int G>
__device__ __forceinline__ void store_f32_frag(float* row, int part, const float (&x)[DL],
                                               float scale) {
  float4* p = reinterpret_cast<float4*>(row);
#pragma unroll
  for (int t = 0; t < DL / 4; ++t)
    p[frag_f4<CH, G>(part, t)] = make_float4(x[4 * t] * scale, x[4 * t + 1] * scale,
                                             x[4 * t + 2] * scale, x[4 * t + 3] * scale);
}

// Stores (x - c * y) * scale as fp32.
template <int DL, int CH, int G>
__device__ __forceinline__ void store_f32_frag_diff(float* row, int part, const float (&x)[DL],
                                                    float c, const float (&y)[DL], float scale) {
  float4* p = reinterpret_cast<float4*>(row);
#pragma unroll
  for (int t = 0; t < DL / 4; ++t) {
    float r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_fmaf(-c, y[4 * t + u], x[4 * t + u]) * scale;
    p[frag_f4<CH, G>(part, t)] = make_float4(r[0], r[1], r[2], r[3]);
  }
}

// Query row j, one key kk: D_j += P dP, A += P dP K, Bv += P K.
template <typename T, int D, int G, typename LoadK, typename LoadV>
__device__ __forceinline__ void dq_key(int kk, float scale_log2, float lse2_j,
                                       const uint32_t (&qf)[Geom<T, D, G>::kWPL],
                                       const uint32_t (&dof)[Geom<T, D, G>::kWPL],
                                       float (&acc_a)[Geom<T, D, G>::kDL],
                                       float (&acc_b)[Geom<T, D, G>::kDL], float& d_j,
                                       LoadK load_k, LoadV load_v) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
  load_k(kk, kf);
  load_v(kk, vf);
  const float s = group_sum<G>(M::dot(qf, kf)) * scale_log2;
  const float dp = group_sum<G>(M::dot(dof, vf));
  const float p = fast_exp2(s - lse2_j);
  const float pdp = p * dp;
  d_j += pdp;
  M::axpy2(acc_a, pdp, acc_b, p, kf);
}

// Query row j: accumulates A = sum P dP K and Bv = sum P K; returns D_j.
template <typename T, int D, int G, typename LoadK, typename LoadV>
__device__ __forceinline__ float dq_row(int j, int N, const int* deltas, int nd, float scale_log2,
                                        float lse2_j, const uint32_t (&qf)[Geom<T, D, G>::kWPL],
                                        const uint32_t (&dof)[Geom<T, D, G>::kWPL],
                                        float (&acc_a)[Geom<T, D, G>::kDL],
                                        float (&acc_b)[Geom<T, D, G>::kDL], LoadK load_k,
                                        LoadV load_v) {
  float d_j = 0.f;
  for (int i = 0; i < nd; ++i) {
    const int kk = j + deltas[i];
    if (kk < 0 || kk >= N) continue;
    dq_key<T, D, G>(kk, scale_log2, lse2_j, qf, dof, acc_a, acc_b, d_j, load_k, load_v);
  }
  return d_j;
}

// Key row kr, one query jj: dV += P dO_jj, dK += P (dP - D_jj) Q_jj.
template <typename T, int D, int G, typename LoadQ, typename LoadDO, typename LoadRow>
__device__ __forceinline__ void dkdv_query(int jj, float scale_log2,
                                           const uint32_t (&kf)[Geom<T, D, G>::kWPL],
                                           const uint32_t (&vf)[Geom<T, D, G>::kWPL],
                                           float (&dk)[Geom<T, D, G>::kDL],
                                           float (&dv)[Geom<T, D, G>::kDL], LoadQ load_q,
                                           LoadDO load_do, LoadRow load_row) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
  load_q(jj, qf);
  load_do(jj, dof);
  float lse2_j, d_j;
  load_row(jj, lse2_j, d_j);
  const float s = group_sum<G>(M::dot(qf, kf)) * scale_log2;
  const float dp = group_sum<G>(M::dot(dof, vf));
  const float p = fast_exp2(s - lse2_j);
  M::axpy(dv, p, dof);
  M::axpy(dk, p * (dp - d_j), qf);
}

// Key row kr: dK and dV over the queries kr + delta.
template <typename T, int D, int G, typename LoadQ, typename LoadDO, typename LoadRow>
__device__ __forceinline__ void dkdv_row(int kr, int N, const int* deltas, int nd,
                                         float scale_log2,
                                         const uint32_t (&kf)[Geom<T, D, G>::kWPL],
                                         const uint32_t (&vf)[Geom<T, D, G>::kWPL],
                                         float (&dk)[Geom<T, D, G>::kDL],
                                         float (&dv)[Geom<T, D, G>::kDL], LoadQ load_q,
                                         LoadDO load_do, LoadRow load_row) {
  for (int i = 0; i < nd; ++i) {
    const int jj = kr + deltas[i];
    if (jj < 0 || jj >= N) continue;
    dkdv_query<T, D, G>(jj, scale_log2, kf, vf, dk, dv, load_q, load_do, load_row);
  }
}

// CLS: class-token mask.  Row 0's dQ and D_0 come from the dense
// class-token kernel (D_0 through the workspace), key 0's dK and dV from the
// dense column kernel, which reads every D_j from the workspace; a row j >= 1
// whose distance to token 0 is not a head distance also pairs with token 0.
template <typename T, int D, int G, int NT, int MH, bool CLS>
__global__ void __launch_bounds__(NT) bwd_slab_kernel(BwdArgs<MH> a) {
  using Gm = Geom<T, D, G>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  const int part = tid % G;
  const Rows rq = slab_rows<T>(a.q, a.lq, slab, a.H), rk = slab_rows<T>(a.k, a.lk, slab, a.H);
  const Rows rv = slab_rows<T>(a.v, a.lv, slab, a.H), rdo = slab_rows<T>(a.dout, a.ldo, slab, a.H);
  const Rows rdq = slab_rows<float>(a.dq, a.ldq, slab, a.H);
  const Rows rdk = slab_rows<float>(a.dk, a.ldk, slab, a.H);
  const Rows rdv = slab_rows<float>(a.dv, a.ldv, slab, a.H);
  char* lds_a = smem;
  char* lds_b = smem + N * Gm::kRowBytes;
  float* s_lse2 = reinterpret_cast<float*>(smem + 2 * N * Gm::kRowBytes);
  float* s_d = s_lse2 + N;

  if (tid == 0) build_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  // The first query row's Q and dO are requested before the staging
  // barrier, so their latency overlaps it.
  const int j0 = tid / G;
  uint32_t qf0[Gm::kWPL], dof0[Gm::kWPL];
  if (j0 < N) {
    frag_load_cached<T, D, G>(rq.row(j0), part, qf0);
    frag_load_cached<T, D, G>(rdo.row(j0), part, dof0);
  }
  stage2_rows_lds<T, D, NT, false>(lds_a, rk.base, rk.rs, lds_b, rv.base, rv.rs, N, tid);
  __syncthreads();
  const int nd = s_nd;

  // Query-centric pass: D_j and dQ_j.
  for (int j = j0; j < N; j += NT / G) {
    const float lse2_j = a.lse[slab * N + j] * kLog2e;
    if (CLS && j == 0) {
      if (part == 0) {
        s_d[0] = a.ws[slab * N];
        s_lse2[0] = lse2_j;
      }
      continue;
    }
    uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
    if (j == j0) {
#pragma unroll
      for (int u = 0; u < Gm::kWPL; ++u) {
        qf[u] = qf0[u];
        dof[u] = dof0[u];
      }
    } else {
      frag_load_cached<T, D, G>(rq.row(j), part, qf);
      frag_load_cached<T, D, G>(rdo.row(j), part, dof);
    }
    float acc_a[Gm::kDL], acc_b[Gm::kDL];
    zero_acc(acc_a);
    zero_acc(acc_b);
    auto lk = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_a, r, part, f); };
    auto lv = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_b, r, part, f); };
    float d_j =
        dq_row<T, D, G>(j, N, s_deltas, nd, a.scale_log2, lse2_j, qf, dof, acc_a, acc_b, lk, lv);
    if (CLS && !has_delta(s_deltas, nd, j))
      dq_key<T, D, G>(0, a.scale_log2, lse2_j, qf, dof, acc_a, acc_b, d_j, lk, lv);
    if (part == 0) {
      s_d[j] = d_j;
      s_lse2[j] = lse2_j;
      if (CLS) a.ws[slab * N + j] = d_j;
    }
    store_f32_frag_diff<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(reinterpret_cast<float*>(rdq.row(j)), part, acc_a, d_j, acc_b,
                                 a.scale);
  }
  // The first key row's K and V come from LDS while they are still there.
  const int k0 = tid / G;
  uint32_t kf0[Gm::kWPL], vf0[Gm::kWPL];
  if (k0 < N) {
    frag_load_lds<T, D, G>(lds_a, k0, part, kf0);
    frag_load_lds<T, D, G>(lds_b, k0, part, vf0);
  }
  __syncthreads();

  // Key-centric pass: Q and dO replace K and V in LDS.
  stage2_rows_lds<T, D, NT, true>(lds_a, rq.base, rq.rs, lds_b, rdo.base, rdo.rs, N, tid);
  __syncthreads();
  for (int kr = k0; kr < N; kr += NT / G) {
    if (CLS && kr == 0) continue;
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    if (kr == k0) {
#pragma unroll
      for (int u = 0; u < Gm::kWPL; ++u) {
        kf[u] = kf0[u];
        vf[u] = vf0[u];
      }
    } else {
      frag_load_cached<T, D, G>(rk.row(kr), part, kf);
      frag_load_cached<T, D, G>(rv.row(kr), part, vf);
    }
    float dk[Gm::kDL], dv[Gm::kDL];
    zero_acc(dk);
    zero_acc(dv);
    auto lq = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_a, r, part, f); };
    auto ldo = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_b, r, part, f); };
    auto lrow = [&](int r, float& l2, float& dd) {
      l2 = s_lse2[r];
      dd = s_d[r];
    };
    dkdv_row<T, D, G>(kr, N, s_deltas, nd, a.scale_log2, kf, vf, dk, dv, lq, ldo, lrow);
    if (CLS && !has_delta(s_deltas, nd, kr))
      dkdv_query<T, D, G>(0, a.scale_log2, kf, vf, dk, dv, lq, ldo, lrow);
    store_f32_frag<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(reinterpret_cast<float*>(rdk.row(kr)), part, dk, a.scale);
    store_f32_frag<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(reinterpret_cast<float*>(rdv.row(kr)), part, dv, 1.0f);
  }
}

// Stream variant, query launch: dQ and D for a tile of query rows.
template <typename T, int D, int G, int NT, int MH, bool CLS>
__global__ void __launch_bounds__(NT) bwd_dq_stream_kernel(BwdArgs<MH> a) {
  using Gm = Geom<T, D, G>;
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.tiles;
  const int tile = blockIdx.x % a.tiles;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  if (tid == 0) build_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  __syncthreads();
  const int j = tile * (NT / G) + tid / G;
  if (j >= N || (CLS && j == 0)) return;
  const int part = tid % G;
  const Rows rk = slab_rows<T>(a.k, a.lk, slab, a.H), rv = slab_rows<T>(a.v, a.lv, slab, a.H);
  uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
  frag_load_cached<T, D, G>(slab_rows<T>(a.q, a.lq, slab, a.H).row(j), part, qf);
  frag_load_cached<T, D, G>(slab_rows<T>(a.dout, a.ldo, slab, a.H).row(j), part, dof);
  const float lse2_j = a.lse[slab * N + j] * kLog2e;
  float acc_a[Gm::kDL], acc_b[Gm::kDL];
  zero_acc(acc_a);
  zero_acc(acc_b);
  auto lk = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(rk.row(r), part, f); };
  auto lv = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(rv.row(r), part, f); };
  float d_j =
      dq_row<T, D, G>(j, N, s_deltas, s_nd, a.scale_log2, lse2_j, qf, dof, acc_a, acc_b, lk, lv);
  if (CLS && !has_delta(s_deltas, s_nd, j))
    dq_key<T, D, G>(0, a.scale_log2, lse2_j, qf, dof, acc_a, acc_b, d_j, lk, lv);
  if (part == 0) a.ws[slab * N + j] = d_j;
  store_f32_frag_diff<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(
      reinterpret_cast<float*>(slab_rows<float>(a.dq, a.ldq, slab, a.H).row(j)), part, acc_a, d_j,
      acc_b, a.scale);
}

// Stream variant, key launch: dK and dV for a tile of key rows.
template <typename T, int D, int G, int NT, int MH, bool CLS>
__global__ void __launch_bounds__(NT) bwd_dkdv_stream_kernel(BwdArgs<MH> a) {
  using Gm = Geom<T, D, G>;
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.tiles;
  const int tile = blockIdx.x % a.tiles;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  if (tid == 0) build_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  __syncthreads();
  const int kr = tile * (NT / G) + tid / G;
  if (kr >= N || (CLS && kr == 0)) return;
  const int part = tid % G;
  const size_t rbase = slab * N;
  const Rows rq = slab_rows<T>(a.q, a.lq, slab, a.H), rdo = slab_rows<T>(a.dout, a.ldo, slab, a.H);
  uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
  frag_load_cached<T, D, G>(slab_rows<T>(a.k, a.lk, slab, a.H).row(kr), part, kf);
  frag_load_cached<T, D, G>(slab_rows<T>(a.v, a.lv, slab, a.H).row(kr), part, vf);
  float dk[Gm::kDL], dv[Gm::kDL];
  zero_acc(dk);
  zero_acc(dv);
  auto lq = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(rq.row(r), part, f); };
  auto ldo = [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(rdo.row(r), part, f); };
  auto lrow = [&](int r, float& l2, float& dd) {
    l2 = a.lse[rbase + r] * kLog2e;
    dd = a.ws[rbase + r];
  };
  dkdv_row<T, D, G>(kr, N, s_deltas, s_nd, a.scale_log2, kf, vf, dk, dv, lq, ldo, lrow);
  if (CLS && !has_delta(s_deltas, s_nd, kr))
    dkdv_query<T, D, G>(0, a.scale_log2, kf, vf, dk, dv, lq, ldo, lrow);
  store_f32_frag<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(
      reinterpret_cast<float*>(slab_rows<float>(a.dk, a.ldk, slab, a.H).row(kr)), part, dk, a.scale);
  store_f32_frag<Gm::kDL, 16 / static_cast<int>(sizeof(T)), G>(
      reinterpret_cast<float*>(slab_rows<float>(a.dv, a.ldv, slab, a.H).row(kr)), part, dv, 1.0f);
}

// Each lane owns 64 bytes of an input row: the key-centric loop keeps two
// row fragments and two fp32 accumulators live, plus two streamed rows.
template <typename T, int D>
constexpr int bwd_group() {
  return (D * static_cast<int>(sizeof(T))) / 64;
}

template <typename T, int D, int MH, bool CLS>
hipError_t launch_bwd_t(const Problem& p, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        float* ws, hipStream_t stream, Path path) {
  constexpr int G = bwd_group<T, D>();
  constexpr int NT = 256;
  using Gm = Geom<T, D, G>;
  BwdArgs<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.dout = static_cast<const char*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = ws;
  a.H = p.H;
  a.N = p.N;
  a.scale = 1.0f / sqrtf(static_cast<float>(D));
  a.scale_log2 = kLog2e * a.scale;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.ldo = p.ldo;
  a.ldq = p.ldq;
  a.ldk = p.ldk;
  a.ldv = p.ldv;
  a.ht = shrink_heads<MH>(p.heads, p.H);
  const size_t slabs = static_cast<size_t>(p.B) * p.H;
  const bool slab_ok = bwd_slab_fits(p);
  if (path == Path::kSlab || (path == Path::kAuto && slab_ok)) {
    if (!slab_ok) return hipErrorInvalidValue;
    const size_t lds = 2 * static_cast<size_t>(p.N) * Gm::kRowBytes + 8 * static_cast<size_t>(p.N);
    constexpr int NTS = 512;  // as the forward's slab kernel
    auto kern = bwd_slab_kernel<T, D, G, NTS, MH, CLS>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        kSlabLdsBudget);
    if (attr != hipSuccess) return attr;
    a.tiles = 1;
    launch(kern, dim3(static_cast<unsigned>(slabs)), dim3(NTS), lds, stream, a);
  } else {
    const int per = NT / G;
    a.tiles = (p.N + per - 1) / per;
    const unsigned blocks = static_cast<unsigned>(slabs * a.tiles);
    launch((bwd_dq_stream_kernel<T, D, G, NT, MH, CLS>), dim3(blocks), dim3(NT), 0, stream, a);
    launch((bwd_dkdv_stream_kernel<T, D, G, NT, MH, CLS>), dim3(blocks), dim3(NT), 0, stream,
                       a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_d(const Problem& p, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        float* ws, hipStream_t stream, Path path) {
  if (p.cls) {
    if (p.H <= kSmallHeads)
      return launch_bwd_t<T, D, kSmallHeads, true>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream,
                                                   path);
    return launch_bwd_t<T, D, kMaxHeads, true>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream,
                                               path);
  }
  if (p.H <= kSmallHeads)
    return launch_bwd_t<T, D, kSmallHeads, false>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream,
                                                  path);
  return launch_bwd_t<T, D, kMaxHeads, false>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
}

}  // namespace

bool bwd_slab_fits(const Problem& p) {
  const int esize = p.dtype == DType::kBF16 ? 2 : 4;
  return 2ll * p.N * p.D * esize + 8ll * p.N <= kSlabLdsBudget;
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      float* ws, hipStream_t stream, Path path) {
  if (path == Path::kAuto && bwd_slab_bf16_fits(p))
    return launch_bwd_slab_bf16(p, q, k, v, lse, dout, dq, dk, dv,
                                p.cls ? cls_discard(p, ws) : nullptr, stream);
  if (path == Path::kAuto && bwd_tile_bf16_fits(p))
    return launch_bwd_tile_bf16(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
  if (p.dtype == DType::kBF16) {
    if (p.D == 64)
      return launch_bwd_d<bf16_t, 64>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
    if (p.D == 128)
      return launch_bwd_d<bf16_t, 128>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
  } else {
    if (p.D == 64)
      return launch_bwd_d<float, 64>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
    if (p.D == 128)
      return launch_bwd_d<float, 128>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
  }
  return hipErrorInvalidValue;
}

}  // namespace fibatt
