// Class-token (CLS) row and column of the Fibottention mask.
//
// The project README's Algorithm 2 builds each head's mask over the class
// token plus N patches: ones everywhere, with the Fibonacci pattern of the
// patches copied into rows and columns 1..N.  So the class token (token 0
// here) attends every token, and every token attends it, on top of the head's
// distance set among the other tokens.
//
// The general kernels handle rows and keys 1..N-1 (each of them pairs with
// token 0 once more when its distance to token 0 is not a head distance).
// This file holds the dense parts, which involve every token of a slab:
//  * forward row 0: softmax of Q_0 . K_k over all k, O_0 = sum_k P_0k V_k;
//  * backward row 0: D_0 = sum_k P_0k dP_0k and dQ_0 = sum_k dS_0k K_k;
//  * backward column 0: dV_0 = sum_j P_j0 dO_j, dK_0 = sum_j dS_j0 Q_j.
// A slab's N rows are split into ranges of kSplitRows; one workgroup reduces
// one range (each lane group walks every NG-th row of it and the groups are
// combined in LDS in a fixed order), and with more than one range a second
// kernel combines the per-range partials, again in a fixed order, so results
// are bitwise reproducible.
#include "kernel_common.h"
#include "launch.h"

namespace fibatt {
namespace {

constexpr int kClsThreads = 256;

struct ClsArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  char* o;       // forward output (row 0 written)
  float* lse;    // forward: row 0 written; backward: read
  float* dq;     // backward outputs (row 0 written)
  float* dk;
  float* dv;
  float* ws_d;   // D per row, [slabs, N]
  float* part;   // per-range partials
  int N;
  int splits;    // ranges per slab
  float scale_log2;
  float scale;
};

// Lane-group width: 64 bytes of a row per lane.
template <typename T, int D>
constexpr int cls_group() {
  return (D * static_cast<int>(sizeof(T))) / 64;
}

template <typename T>
__device__ __forceinline__ void store_elem(char* row, int e, float x) {
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<uint16_t*>(row)[e] = static_cast<uint16_t>(f32_to_bf16(x));
  } else {
    reinterpret_cast<float*>(row)[e] = x;
  }
}

// Sums x (each group's kDL elements of a D-vector) over the workgroup's
// groups in group order; thread t < D receives element t.  `buf` holds
// NG * D floats.
template <int D, int G, int NT>
__device__ __forceinline__ float groups_sum(float* buf, int tid, const float* x) {
  constexpr int kDL = D / G;
  const int g = tid / G, part = tid % G;
#pragma unroll
  for (int t = 0; t < kDL; ++t) buf[g * D + part * kDL + t] = x[t];
  __syncthreads();
  float s = 0.f;
  if (tid < D)
    for (int i = 0; i < NT / G; ++i) s += buf[i * D + tid];
  __syncthreads();
  return s;
}

template <int NG>
__device__ __forceinline__ float scalar_sum(const float* buf) {
  float s = 0.f;
  for (int i = 0; i < NG; ++i) s += buf[i];
  return s;
}

// Forward, row 0 against the keys of one range.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) fwd_cls_row_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int NG = NT / G;
  constexpr int C = 4;
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  __shared__ float s_buf[NG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int k0 = sp * kSplitRows;
  const int k1 = min(N, k0 + kSplitRows);
  const int g = tid / G, part = tid % G;
  const size_t base = slab * N * Gm::kRowBytes;
  uint32_t qf[Gm::kWPL];
  frag_load_cached<T, D, G>(a.q + base, part, qf);
  float acc[Gm::kDL];
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) acc[t] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int c0 = k0 + g; c0 < k1; c0 += NG * C) {
    float s[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int kk = c0 + c * NG;
      s[c] = -INFINITY;
      if (kk < k1) {
        uint32_t kf[Gm::kWPL];
        frag_load_cached<T, D, G>(a.k + base + static_cast<size_t>(kk) * Gm::kRowBytes, part, kf);
        s[c] = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
      }
    }
    float mc = s[0];
#pragma unroll
    for (int c = 1; c < C; ++c) mc = fmaxf(mc, s[c]);
    const float mn = fmaxf(m, mc);  // finite: key c0 is in range
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < Gm::kDL; ++t) acc[t] *= alpha;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int kk = c0 + c * NG;
      if (kk < k1) {
        const float p = fast_exp2(s[c] - mn);
        l += p;
        uint32_t vf[Gm::kWPL];
        frag_load_cached<T, D, G>(a.v + base + static_cast<size_t>(kk) * Gm::kRowBytes, part, vf);
        M::axpy(acc, p, vf);
      }
    }
    m = mn;
  }
  // Combine the groups: common maximum, rescaled sums.
  if (part == 0) s_m[g] = m;
  __syncthreads();
  float mx = -INFINITY;
  for (int i = 0; i < NG; ++i) mx = fmaxf(mx, s_m[i]);  // group 0 always has a key
  const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mx);
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) acc[t] *= alpha;
  if (part == 0) s_l[g] = l * alpha;
  const float o = groups_sum<D, G, NT>(s_buf, tid, acc);
  const float lsum = scalar_sum<NG>(s_l);
  if (tid < D) {
    if (a.splits == 1) {
      store_elem<T>(a.o + base, tid, o / lsum);
      if (tid == 0) a.lse[slab * N] = (mx + fast_log2(lsum)) * kLn2;
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (D + 2);
      pp[2 + tid] = o;
      if (tid == 0) {
        pp[0] = mx;
        pp[1] = lsum;
      }
    }
  }
}

// Forward, combination of a slab's ranges (one thread per element).
template <typename T, int D>
__global__ void __launch_bounds__(D) fwd_cls_combine_kernel(ClsArgs a) {
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const float* pp = a.part + slab * a.splits * (D + 2);
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, pp[s * (D + 2)]);
  float lsum = 0.f, o = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float w = fast_exp2(pp[s * (D + 2)] - mx);
    lsum = __builtin_fmaf(pp[s * (D + 2) + 1], w, lsum);
    o = __builtin_fmaf(pp[s * (D + 2) + 2 + tid], w, o);
  }
  const size_t row_bytes = static_cast<size_t>(D) * sizeof(T);
  store_elem<T>(a.o + slab * a.N * row_bytes, tid, o / lsum);
  if (tid == 0) a.lse[slab * a.N] = (mx + fast_log2(lsum)) * kLn2;
}

// Backward, row 0 against the keys of one range: D_0 and dQ_0 = (A - D_0 Bv)
// scale with A = sum P dP K and Bv = sum P K.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_cls_row_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int NG = NT / G;
  __shared__ float s_d[NG];
  __shared__ float s_buf[NG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int k0 = sp * kSplitRows;
  const int k1 = min(N, k0 + kSplitRows);
  const int g = tid / G, part = tid % G;
  const size_t base = slab * N * Gm::kRowBytes;
  uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
  frag_load_cached<T, D, G>(a.q + base, part, qf);
  frag_load_cached<T, D, G>(a.dout + base, part, dof);
  const float lse2 = a.lse[slab * N] * kLog2e;
  float acc_a[Gm::kDL], acc_b[Gm::kDL];
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) acc_a[t] = acc_b[t] = 0.f;
  float d = 0.f;
  for (int kk = k0 + g; kk < k1; kk += NG) {
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    frag_load_cached<T, D, G>(a.k + base + static_cast<size_t>(kk) * Gm::kRowBytes, part, kf);
    frag_load_cached<T, D, G>(a.v + base + static_cast<size_t>(kk) * Gm::kRowBytes, part, vf);
    const float s = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
    const float dp = group_sum<G>(M::dot(dof, vf));
    const float p = fast_exp2(s - lse2);
    d = __builtin_fmaf(p, dp, d);
    M::axpy2(acc_a, p * dp, acc_b, p, kf);
  }
  if (part == 0) s_d[g] = d;
  const float A = groups_sum<D, G, NT>(s_buf, tid, acc_a);
  const float Bv = groups_sum<D, G, NT>(s_buf, tid, acc_b);
  const float dsum = scalar_sum<NG>(s_d);
  if (tid < D) {
    if (a.splits == 1) {
      a.dq[slab * N * D + tid] = __builtin_fmaf(-dsum, Bv, A) * a.scale;
      if (tid == 0) a.ws_d[slab * N] = dsum;
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (2 * D + 1);
      pp[1 + tid] = A;
      pp[1 + D + tid] = Bv;
      if (tid == 0) pp[0] = dsum;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D) bwd_cls_row_combine_kernel(ClsArgs a) {
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const float* pp = a.part + slab * a.splits * (2 * D + 1);
  float dsum = 0.f, A = 0.f, Bv = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* q = pp + s * (2 * D + 1);
    dsum += q[0];
    A += q[1 + tid];
    Bv += q[1 + D + tid];
  }
  a.dq[slab * a.N * D + tid] = __builtin_fmaf(-dsum, Bv, A) * a.scale;
  if (tid == 0) a.ws_d[slab * a.N] = dsum;
}

// Backward, column 0 against the queries of one range.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_cls_col_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int NG = NT / G;
  __shared__ float s_buf[NG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int j0 = sp * kSplitRows;
  const int j1 = min(N, j0 + kSplitRows);
  const int g = tid / G, part = tid % G;
  const size_t base = slab * N * Gm::kRowBytes;
  uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
  frag_load_cached<T, D, G>(a.k + base, part, kf);
  frag_load_cached<T, D, G>(a.v + base, part, vf);
  float dk[Gm::kDL], dv[Gm::kDL];
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) dk[t] = dv[t] = 0.f;
  for (int jj = j0 + g; jj < j1; jj += NG) {
    uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
    frag_load_cached<T, D, G>(a.q + base + static_cast<size_t>(jj) * Gm::kRowBytes, part, qf);
    frag_load_cached<T, D, G>(a.dout + base + static_cast<size_t>(jj) * Gm::kRowBytes, part, dof);
    const float lse2 = a.lse[slab * N + jj] * kLog2e;
    const float dj = a.ws_d[slab * N + jj];
    const float s = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
    const float dp = group_sum<G>(M::dot(dof, vf));
    const float p = fast_exp2(s - lse2);
    M::axpy(dv, p, dof);
    M::axpy(dk, p * (dp - dj), qf);
  }
  const float sk = groups_sum<D, G, NT>(s_buf, tid, dk);
  const float sv = groups_sum<D, G, NT>(s_buf, tid, dv);
  if (tid < D) {
    if (a.splits == 1) {
      a.dk[slab * N * D + tid] = sk * a.scale;
      a.dv[slab * N * D + tid] = sv;
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (2 * D);
      pp[tid] = sk;
      pp[D + tid] = sv;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D) bwd_cls_col_combine_kernel(ClsArgs a) {
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const float* pp = a.part + slab * a.splits * (2 * D);
  float sk = 0.f, sv = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    sk += pp[s * 2 * D + tid];
    sv += pp[s * 2 * D + D + tid];
  }
  a.dk[slab * a.N * D + tid] = sk * a.scale;
  a.dv[slab * a.N * D + tid] = sv;
}

ClsArgs make_args(const Problem& p) {
  ClsArgs a{};
  a.N = p.N;
  a.splits = cls_splits(p);
  a.scale = 1.0f / sqrtf(static_cast<float>(p.D));
  a.scale_log2 = kLog2e * a.scale;
  return a;
}

template <typename T, int D>
hipError_t fwd_row_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  hipLaunchKernelGGL((fwd_cls_row_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    hipLaunchKernelGGL((fwd_cls_combine_kernel<T, D>), dim3(slabs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_row_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  hipLaunchKernelGGL((bwd_cls_row_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    hipLaunchKernelGGL((bwd_cls_row_combine_kernel<D>), dim3(slabs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_col_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  hipLaunchKernelGGL((bwd_cls_col_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    hipLaunchKernelGGL((bwd_cls_col_combine_kernel<D>), dim3(slabs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

#define FIBATT_CLS_DISPATCH(fn, p, a, stream)                                       \
  do {                                                                              \
    if ((p).dtype == DType::kBF16) {                                                \
      if ((p).D == 64) return fn<bf16_t, 64>(p, a, stream);                         \
      if ((p).D == 128) return fn<bf16_t, 128>(p, a, stream);                       \
    } else {                                                                        \
      if ((p).D == 64) return fn<float, 64>(p, a, stream);                          \
      if ((p).D == 128) return fn<float, 128>(p, a, stream);                        \
    }                                                                               \
    return hipErrorInvalidValue;                                                    \
  } while (0)

hipError_t fwd_row(const Problem& p, const ClsArgs& a, hipStream_t stream) {
  FIBATT_CLS_DISPATCH(fwd_row_t, p, a, stream);
}
hipError_t bwd_row(const Problem& p, const ClsArgs& a, hipStream_t stream) {
  FIBATT_CLS_DISPATCH(bwd_row_t, p, a, stream);
}
hipError_t bwd_col(const Problem& p, const ClsArgs& a, hipStream_t stream) {
  FIBATT_CLS_DISPATCH(bwd_col_t, p, a, stream);
}

}  // namespace

int cls_splits(const Problem& p) { return (p.N + kSplitRows - 1) / kSplitRows; }

int64_t fwd_cls_workspace_floats(const Problem& p) {
  const int s = cls_splits(p);
  return s > 1 ? static_cast<int64_t>(p.B) * p.H * s * (p.D + 2) : 0;
}

int64_t bwd_cls_workspace_floats(const Problem& p) {
  const int s = cls_splits(p);
  const int64_t slabs = static_cast<int64_t>(p.B) * p.H;
  return slabs * p.N + (s > 1 ? slabs * s * (2 * p.D + 1) : 0);
}

hipError_t launch_fwd_cls(const Problem& p0, const void* q, const void* k, const void* v,
                          void* o, float* lse, float* ws, hipStream_t stream, Path path) {
  Problem p = p0;
  p.cls = true;
  hipError_t e = launch_fwd(p, q, k, v, o, lse, stream, path);
  if (e != hipSuccess) return e;
  ClsArgs a = make_args(p);
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.part = ws;
  return fwd_row(p, a, stream);
}

hipError_t launch_bwd_cls(const Problem& p0, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv,
                          float* ws, hipStream_t stream, Path path) {
  Problem p = p0;
  p.cls = true;
  ClsArgs a = make_args(p);
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.dout = static_cast<const char*>(dout);
  a.lse = const_cast<float*>(lse);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws_d = ws;
  a.part = ws + static_cast<size_t>(p.B) * p.H * p.N;
  // Row 0 first: the key pass of the general kernels needs D_0.
  hipError_t e = bwd_row(p, a, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
  if (e != hipSuccess) return e;
  // Column 0 last: it needs every D_j.
  return bwd_col(p, a, stream);
}

}  // namespace fibatt
