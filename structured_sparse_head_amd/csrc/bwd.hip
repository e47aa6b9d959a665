// Backward kernels: exact gradients of the sparse Fibottention attention.
//
// The pages define only the forward (Fibottention paper, method section,
// eq. (1) and (3); README Algorithm 3).  The backward is its derivative:
// with P the support-restricted softmax, dP_jk = dO_j . V_k and
// D_j = sum_k P_jk dP_jk = dO_j . O_j,
//   dS_jk = P_jk (dP_jk - D_j),
//   dQ_j  = sum_k dS_jk K_k / sqrt(d),
//   dK_k  = sum_j dS_jk Q_j / sqrt(d),
//   dV_k  = sum_j P_jk dO_j.
// The support is symmetric in j and k (the set is defined through |j - k|),
// so the queries that see key k are exactly k + delta for the same signed
// displacements delta.  dK and dV are therefore gathered key by key over the
// same displacement list: every output row has a single writer, no atomics,
// and the result is bitwise reproducible.  P is recomputed from the forward's
// log-sum-exp (P_jk = exp(S_jk - LSE_j)).
//
// Variants mirror the forward:
//  * slab: one workgroup per (b, h) slab.  K and V are staged into LDS for
//    the query-centric dQ phase (which also produces D_j); then Q and dO
//    replace them for the key-centric dK/dV phase.  LSE and D of the whole
//    slab stay in LDS between the phases.
//  * stream: a pre-pass writes D to the workspace; one launch then runs
//    query-tile workgroups (dQ) and key-tile workgroups (dK, dV) side by
//    side, reading shifted rows straight from global memory.
#include "kernel_common.h"
#include "launch.h"

namespace fibatt {
namespace {

struct BwdArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* ws;
  int H;
  int N;
  int tiles;         // row tiles per slab (stream variant)
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
  HeadTable ht;
};

template <typename T, int D, int G>
__device__ __forceinline__ void store_f32_frag(float* row, int part,
                                               const float (&acc)[Geom<T, D, G>::kDL],
                                               float scale) {
  constexpr int kDL = Geom<T, D, G>::kDL;
  float4* p = reinterpret_cast<float4*>(row) + part * (kDL / 4);
#pragma unroll
  for (int t = 0; t < kDL / 4; ++t)
    p[t] = make_float4(acc[4 * t] * scale, acc[4 * t + 1] * scale, acc[4 * t + 2] * scale,
                       acc[4 * t + 3] * scale);
}

template <int DL>
__device__ __forceinline__ void zero_acc(float* acc) {
#pragma unroll
  for (int t = 0; t < DL; ++t) acc[t] = 0.f;
}

// One query row's dQ given K/V loaders; returns nothing, accumulates into dq.
template <typename T, int D, int G, typename LoadK, typename LoadV>
__device__ __forceinline__ void dq_row(int j, int N, int part, const int* deltas, int nd,
                                       float scale_log2, float lse2_j, float d_j,
                                       const uint32_t (&qf)[Geom<T, D, G>::kWPL],
                                       const uint32_t (&dof)[Geom<T, D, G>::kWPL],
                                       float (&dq)[Geom<T, D, G>::kDL], LoadK load_k,
                                       LoadV load_v) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  for (int i = 0; i < nd; ++i) {
    const int kk = j + deltas[i];
    if (kk < 0 || kk >= N) continue;
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    load_k(kk, kf);
    load_v(kk, vf);
    const float s = group_sum<G>(M::dot(qf, kf)) * scale_log2;
    const float dp = group_sum<G>(M::dot(dof, vf));
    const float p = fast_exp2(s - lse2_j);
    M::axpy(dq, p * (dp - d_j), kf);
  }
}

// One key row's dK, dV given Q/dO/LSE/D loaders.
template <typename T, int D, int G, typename LoadQ, typename LoadDO, typename LoadRow>
__device__ __forceinline__ void dkdv_row(int kr, int N, const int* deltas, int nd,
                                         float scale_log2,
                                         const uint32_t (&kf)[Geom<T, D, G>::kWPL],
                                         const uint32_t (&vf)[Geom<T, D, G>::kWPL],
                                         float (&dk)[Geom<T, D, G>::kDL],
                                         float (&dv)[Geom<T, D, G>::kDL], LoadQ load_q,
                                         LoadDO load_do, LoadRow load_row) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  for (int i = 0; i < nd; ++i) {
    const int jj = kr + deltas[i];
    if (jj < 0 || jj >= N) continue;
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
}

template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_slab_kernel(BwdArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  const int part = tid % G;
  const size_t base = slab * N * Gm::kRowBytes;
  const size_t fbase = slab * N * D;  // fp32 outputs, elements
  char* lds_a = smem;
  char* lds_b = smem + N * Gm::kRowBytes;
  float* s_lse2 = reinterpret_cast<float*>(smem + 2 * N * Gm::kRowBytes);
  float* s_d = s_lse2 + N;

  if (tid == 0) build_deltas(a.ht.a[h], a.ht.b[h], a.ht.lim[h], s_dist, s_deltas, &s_nd);
  stage_rows_lds<T, D, NT, false>(lds_a, a.k + base, N, tid);
  stage_rows_lds<T, D, NT, false>(lds_b, a.v + base, N, tid);
  __syncthreads();
  const int nd = s_nd;

  // Query-centric phase: D_j, then dQ_j.
  for (int j = tid / G; j < N; j += NT / G) {
    const size_t roff = base + static_cast<size_t>(j) * Gm::kRowBytes;
    uint32_t qf[Gm::kWPL], dof[Gm::kWPL], of[Gm::kWPL];
    frag_load_cached<T, D, G>(a.q + roff, part, qf);
    frag_load_cached<T, D, G>(a.dout + roff, part, dof);
    frag_load_global<T, D, G>(a.o + roff, part, of);
    const float d_j = group_sum<G>(M::dot(dof, of));
    const float lse2_j = a.lse[slab * N + j] * kLog2e;
    if (part == 0) {
      s_d[j] = d_j;
      s_lse2[j] = lse2_j;
    }
    float dq[Gm::kDL];
    zero_acc<Gm::kDL>(dq);
    dq_row<T, D, G>(
        j, N, part, s_deltas, nd, a.scale_log2, lse2_j, d_j, qf, dof, dq,
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_a, r, part, f); },
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_b, r, part, f); });
    store_f32_frag<T, D, G>(a.dq + fbase + static_cast<size_t>(j) * D, part, dq, a.scale);
  }
  __syncthreads();

  // Key-centric phase: Q and dO replace K and V in LDS.
  stage_rows_lds<T, D, NT, true>(lds_a, a.q + base, N, tid);
  stage_rows_lds<T, D, NT, true>(lds_b, a.dout + base, N, tid);
  __syncthreads();
  for (int kr = tid / G; kr < N; kr += NT / G) {
    const size_t roff = base + static_cast<size_t>(kr) * Gm::kRowBytes;
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    frag_load_cached<T, D, G>(a.k + roff, part, kf);
    frag_load_cached<T, D, G>(a.v + roff, part, vf);
    float dk[Gm::kDL], dv[Gm::kDL];
    zero_acc<Gm::kDL>(dk);
    zero_acc<Gm::kDL>(dv);
    dkdv_row<T, D, G>(
        kr, N, s_deltas, nd, a.scale_log2, kf, vf, dk, dv,
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_a, r, part, f); },
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_lds<T, D, G>(lds_b, r, part, f); },
        [&](int r, float& l2, float& dd) {
          l2 = s_lse2[r];
          dd = s_d[r];
        });
    store_f32_frag<T, D, G>(a.dk + fbase + static_cast<size_t>(kr) * D, part, dk, a.scale);
    store_f32_frag<T, D, G>(a.dv + fbase + static_cast<size_t>(kr) * D, part, dv, 1.0f);
  }
}

// D_j = dO_j . O_j for every row (stream variant).
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_pre_kernel(BwdArgs a, size_t rows) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  const size_t r = static_cast<size_t>(blockIdx.x) * (NT / G) + threadIdx.x / G;
  if (r >= rows) return;
  const int part = threadIdx.x % G;
  uint32_t of[Gm::kWPL], dof[Gm::kWPL];
  frag_load_global<T, D, G>(a.o + r * Gm::kRowBytes, part, of);
  frag_load_cached<T, D, G>(a.dout + r * Gm::kRowBytes, part, dof);
  const float d = group_sum<G>(M::dot(dof, of));
  if (part == 0) a.ws[r] = d;
}

// Stream variant: blocks [0, S*tiles) compute dQ for a query tile, blocks
// [S*tiles, 2*S*tiles) compute dK/dV for a key tile.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_stream_kernel(BwdArgs a, unsigned dq_blocks) {
  using Gm = Geom<T, D, G>;
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const bool key_role = blockIdx.x >= dq_blocks;
  const unsigned bid = key_role ? blockIdx.x - dq_blocks : blockIdx.x;
  const size_t slab = bid / a.tiles;
  const int tile = bid % a.tiles;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  if (tid == 0) build_deltas(a.ht.a[h], a.ht.b[h], a.ht.lim[h], s_dist, s_deltas, &s_nd);
  __syncthreads();
  const int row = tile * (NT / G) + tid / G;
  if (row >= N) return;
  const int part = tid % G;
  const int nd = s_nd;
  const size_t base = slab * N * Gm::kRowBytes;
  const size_t rbase = slab * N;
  const size_t fbase = slab * N * D;
  const char* qs = a.q + base;
  const char* ks = a.k + base;
  const char* vs = a.v + base;
  const char* dos = a.dout + base;
  auto row_ptr = [](const char* s, int r) { return s + static_cast<size_t>(r) * Gm::kRowBytes; };
  if (!key_role) {
    uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
    frag_load_global<T, D, G>(row_ptr(qs, row), part, qf);
    frag_load_cached<T, D, G>(row_ptr(dos, row), part, dof);
    const float lse2_j = a.lse[rbase + row] * kLog2e;
    const float d_j = a.ws[rbase + row];
    float dq[Gm::kDL];
    zero_acc<Gm::kDL>(dq);
    dq_row<T, D, G>(
        row, N, part, s_deltas, nd, a.scale_log2, lse2_j, d_j, qf, dof, dq,
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(row_ptr(ks, r), part, f); },
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(row_ptr(vs, r), part, f); });
    store_f32_frag<T, D, G>(a.dq + fbase + static_cast<size_t>(row) * D, part, dq, a.scale);
  } else {
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    frag_load_cached<T, D, G>(row_ptr(ks, row), part, kf);
    frag_load_cached<T, D, G>(row_ptr(vs, row), part, vf);
    float dk[Gm::kDL], dv[Gm::kDL];
    zero_acc<Gm::kDL>(dk);
    zero_acc<Gm::kDL>(dv);
    dkdv_row<T, D, G>(
        row, N, s_deltas, nd, a.scale_log2, kf, vf, dk, dv,
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(row_ptr(qs, r), part, f); },
        [&](int r, uint32_t(&f)[Gm::kWPL]) { frag_load_cached<T, D, G>(row_ptr(dos, r), part, f); },
        [&](int r, float& l2, float& dd) {
          l2 = a.lse[rbase + r] * kLog2e;
          dd = a.ws[rbase + r];
        });
    store_f32_frag<T, D, G>(a.dk + fbase + static_cast<size_t>(row) * D, part, dk, a.scale);
    store_f32_frag<T, D, G>(a.dv + fbase + static_cast<size_t>(row) * D, part, dv, 1.0f);
  }
}

// Each lane owns 64 bytes of an input row (registers hold four row
// fragments plus two fp32 accumulators in the key-centric loop).
template <typename T, int D>
constexpr int bwd_group() {
  return (D * static_cast<int>(sizeof(T))) / 64;
}

template <typename T, int D>
hipError_t launch_bwd_t(const Problem& p, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout, float* dq, float* dk,
                        float* dv, float* ws, hipStream_t stream, Path path) {
  constexpr int G = bwd_group<T, D>();
  constexpr int NT = 256;
  using Gm = Geom<T, D, G>;
  BwdArgs a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<const char*>(o);
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
  a.ht = p.heads;
  const size_t slabs = static_cast<size_t>(p.B) * p.H;
  const bool slab_ok = bwd_slab_fits(p);
  if (path == Path::kSlab || (path == Path::kAuto && slab_ok)) {
    if (!slab_ok) return hipErrorInvalidValue;
    const size_t lds = 2 * static_cast<size_t>(p.N) * Gm::kRowBytes + 8 * static_cast<size_t>(p.N);
    auto kern = bwd_slab_kernel<T, D, G, NT>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        kSlabLdsBudget);
    if (attr != hipSuccess) return attr;
    a.tiles = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(slabs)), dim3(NT), lds, stream, a);
  } else {
    const size_t rows = slabs * p.N;
    const unsigned pre_blocks = static_cast<unsigned>((rows + NT / G - 1) / (NT / G));
    hipLaunchKernelGGL((bwd_pre_kernel<T, D, G, NT>), dim3(pre_blocks), dim3(NT), 0, stream, a,
                       rows);
    const int per = NT / G;
    a.tiles = (p.N + per - 1) / per;
    const unsigned dq_blocks = static_cast<unsigned>(slabs * a.tiles);
    hipLaunchKernelGGL((bwd_stream_kernel<T, D, G, NT>), dim3(2 * dq_blocks), dim3(NT), 0, stream,
                       a, dq_blocks);
  }
  return hipGetLastError();
}

}  // namespace

bool bwd_slab_fits(const Problem& p) {
  const int esize = p.dtype == DType::kBF16 ? 2 : 4;
  return 2ll * p.N * p.D * esize + 8ll * p.N <= kSlabLdsBudget;
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, float* dq, float* dk,
                      float* dv, float* ws, hipStream_t stream, Path path) {
  if (p.dtype == DType::kBF16) {
    if (p.D == 64)
      return launch_bwd_t<bf16_t, 64>(p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, path);
    if (p.D == 128)
      return launch_bwd_t<bf16_t, 128>(p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, path);
  } else {
    if (p.D == 64)
      return launch_bwd_t<float, 64>(p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, path);
    if (p.D == 128)
      return launch_bwd_t<float, 128>(p, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, path);
  }
  return hipErrorInvalidValue;
}

}  // namespace fibatt
