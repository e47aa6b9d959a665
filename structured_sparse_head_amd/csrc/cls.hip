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
//  * forward row 0: softmax of Q_0 . K_k over all k, O_0 = sum_k P_0k V_k
//    (launched after the main forward, whose row 0 it replaces);
//  * backward row 0: D_0 = sum_k P_0k dP_0k and dQ_0 = sum_k dS_0k K_k
//    (launched first: the main backward reads D_0; dQ_0 waits in the
//    workspace, because the main kernels may write row 0 of dQ);
//  * backward column 0: dV_0 = sum_j P_j0 dO_j, dK_0 = sum_j dS_j0 Q_j
//    (launched last, with every D_j in the workspace; it also copies dQ_0
//    into place).
// The persistent ViT kernels do the dense parts themselves, from the slab in
// LDS (forward for N <= 240, backward always).
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
  float* dq0;    // dQ of row 0 per slab, [slabs, D], copied into dq last
  float* part;   // per-range partials
  int H;
  int N;
  int splits;    // ranges per slab
  float scale_log2;
  float scale;
  Layout lq, lk, lv, lo, ldo, ldq, ldk, ldv;  // row layouts of the tensors
};

// Row r of slab `slab` of tensor x (layout l, es-byte elements).
__device__ __forceinline__ const char* lrow(const char* x, const Layout& l, size_t slab, int H,
                                            int es, int r) {
  return x + l.slab_bytes(slab, H, es) + static_cast<size_t>(r) * l.row_bytes(es);
}
__device__ __forceinline__ float* lrow_f32(float* x, const Layout& l, size_t slab, int H) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(x) + l.slab_bytes(slab, H, 4));
}

// Lane-group width for the per-row dot products: 64 bytes of a row per lane.
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

// Block-wide max and sum of one value per thread: a butterfly inside each
// wave, then the waves in order.  Every thread gets wave 0's lane 0 order.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r += red[i];
  __syncthreads();
  return r;
}

// Weighted sums of n rows of x (rows of D elements of T, rs bytes apart,
// rows r0 ..): out_c[e] = sum_i coef_c[i] x_{r0 + i}[e] for NC coefficient
// arrays (LDS).
// Each thread takes one 16-byte chunk of a row and every KG-th row; the KG
// partial sums of an element are added in order.  Thread e < D gets element
// e; `red` holds KG * D floats.
template <typename T, int D, int NT, int NC>
__device__ __forceinline__ void rows_wsum(const char* x, size_t rs, int r0, int n,
                                          const float* const* coef, float* red,
                                          float (&out)[NC]) {
  constexpr int CH = 16 / static_cast<int>(sizeof(T));  // elements per chunk
  constexpr int CPR = D / CH;                           // chunks per row
  constexpr int KG = NT / CPR;                          // row groups
  const int tid = threadIdx.x;
  const int c = tid % CPR, kg = tid / CPR;
  float acc[NC][CH];
#pragma unroll
  for (int u = 0; u < NC; ++u)
#pragma unroll
    for (int t = 0; t < CH; ++t) acc[u][t] = 0.f;
  const char* base = x + static_cast<size_t>(r0) * rs + c * 16;
#pragma unroll 4
  for (int i = kg; i < n; i += KG) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(i) * rs);
    float e[CH];
    if constexpr (sizeof(T) == 2) {
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e[2 * t] = bf16_lo(ww[t]);
        e[2 * t + 1] = bf16_hi(ww[t]);
      }
    } else {
      e[0] = __uint_as_float(w.x);
      e[1] = __uint_as_float(w.y);
      e[2] = __uint_as_float(w.z);
      e[3] = __uint_as_float(w.w);
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const float cf = coef[u][i];
#pragma unroll
      for (int t = 0; t < CH; ++t) acc[u][t] = __builtin_fmaf(cf, e[t], acc[u][t]);
    }
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
#pragma unroll
    for (int t = 0; t < CH; ++t) red[kg * D + c * CH + t] = acc[u][t];
    __syncthreads();
    float s = 0.f;
    if (tid < D)
      for (int j = 0; j < KG; ++j) s += red[j * D + tid];
    out[u] = s;
    __syncthreads();
  }
}

// Per-row dot products of one range: group g (G lanes) takes rows r0 + g,
// r0 + g + NG, ...; f(i, r, part) runs for each with the group's lanes.
template <int G, int NT, typename F>
__device__ __forceinline__ void for_rows(int r0, int r1, F f) {
  const int g = threadIdx.x / G, part = threadIdx.x % G;
  for (int r = r0 + g; r < r1; r += NT / G) f(r - r0, r, part);
}

// Forward, row 0 against the keys of one range.  Scores in base 2; the
// range's (max, sum of exp, sum of exp V) are final or a partial.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) fwd_cls_row_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int KG = NT / (D * static_cast<int>(sizeof(T)) / 16);
  __shared__ float s_w[kSplitRows];
  __shared__ float s_red[KG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int k0 = sp * kSplitRows;
  const int k1 = min(N, k0 + kSplitRows);
  const int n = k1 - k0;
  constexpr int es = sizeof(T);
  const char* ks = lrow(a.k, a.lk, slab, a.H, es, 0);
  const size_t rk = a.lk.row_bytes(es);
  uint32_t qf[Gm::kWPL];
  frag_load_cached<T, D, G>(lrow(a.q, a.lq, slab, a.H, es, 0), tid % G, qf);
  for_rows<G, NT>(k0, k1, [&](int i, int r, int part) {
    uint32_t kf[Gm::kWPL];
    frag_load_cached<T, D, G>(ks + static_cast<size_t>(r) * rk, part, kf);
    const float s = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
    if (part == 0) s_w[i] = s;
  });
  __syncthreads();
  float m = -INFINITY;
  for (int i = tid; i < n; i += NT) m = fmaxf(m, s_w[i]);
  m = block_max<NT>(m, s_red);
  float l = 0.f;
  for (int i = tid; i < n; i += NT) {
    const float w = fast_exp2(s_w[i] - m);
    s_w[i] = w;
    l += w;
  }
  l = block_sum<NT>(l, s_red);  // (its barrier also publishes s_w)
  const float* coef[1] = {s_w};
  float o[1];
  rows_wsum<T, D, NT, 1>(lrow(a.v, a.lv, slab, a.H, es, 0), a.lv.row_bytes(es), k0, n, coef,
                         s_red, o);
  if (tid < D) {
    if (a.splits == 1) {
      store_elem<T>(const_cast<char*>(lrow(a.o, a.lo, slab, a.H, es, 0)), tid, o[0] / l);
      if (tid == 0) a.lse[slab * N] = (m + fast_log2(l)) * kLn2;
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (D + 2);
      pp[2 + tid] = o[0];
      if (tid == 0) {
        pp[0] = m;
        pp[1] = l;
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
  store_elem<T>(const_cast<char*>(lrow(a.o, a.lo, slab, a.H, sizeof(T), 0)), tid, o / lsum);
  if (tid == 0) a.lse[slab * a.N] = (mx + fast_log2(lsum)) * kLn2;
}

// Backward, row 0 against the keys of one range: D_0 and dQ_0 = (A - D_0 Bv)
// scale with A = sum P dP K and Bv = sum P K.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_cls_row_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int KG = NT / (D * static_cast<int>(sizeof(T)) / 16);
  __shared__ float s_pdp[kSplitRows];
  __shared__ float s_p[kSplitRows];
  __shared__ float s_red[KG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int k0 = sp * kSplitRows;
  const int k1 = min(N, k0 + kSplitRows);
  const int n = k1 - k0;
  constexpr int es = sizeof(T);
  const char* ks = lrow(a.k, a.lk, slab, a.H, es, 0);
  const char* vs = lrow(a.v, a.lv, slab, a.H, es, 0);
  const size_t rk = a.lk.row_bytes(es), rv = a.lv.row_bytes(es);
  uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
  frag_load_cached<T, D, G>(lrow(a.q, a.lq, slab, a.H, es, 0), tid % G, qf);
  frag_load_cached<T, D, G>(lrow(a.dout, a.ldo, slab, a.H, es, 0), tid % G, dof);
  const float lse2 = a.lse[slab * N] * kLog2e;
  for_rows<G, NT>(k0, k1, [&](int i, int r, int part) {
    uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
    frag_load_cached<T, D, G>(ks + static_cast<size_t>(r) * rk, part, kf);
    frag_load_cached<T, D, G>(vs + static_cast<size_t>(r) * rv, part, vf);
    const float s = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
    const float dp = group_sum<G>(M::dot(dof, vf));
    const float p = fast_exp2(s - lse2);
    if (part == 0) {
      s_pdp[i] = p * dp;
      s_p[i] = p;
    }
  });
  __syncthreads();
  float d = 0.f;
  for (int i = tid; i < n; i += NT) d += s_pdp[i];
  d = block_sum<NT>(d, s_red);
  const float* coef[2] = {s_pdp, s_p};
  float ab[2];
  rows_wsum<T, D, NT, 2>(ks, rk, k0, n, coef, s_red, ab);
  if (tid < D) {
    if (a.splits == 1) {
      a.dq0[slab * D + tid] = __builtin_fmaf(-d, ab[1], ab[0]) * a.scale;
      if (tid == 0) a.ws_d[slab * N] = d;
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (2 * D + 1);
      pp[1 + tid] = ab[0];
      pp[1 + D + tid] = ab[1];
      if (tid == 0) pp[0] = d;
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
  a.dq0[slab * D + tid] = __builtin_fmaf(-dsum, Bv, A) * a.scale;
  if (tid == 0) a.ws_d[slab * a.N] = dsum;
}

// Backward, column 0 against the queries of one range.
template <typename T, int D, int G, int NT>
__global__ void __launch_bounds__(NT) bwd_cls_col_kernel(ClsArgs a) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  constexpr int KG = NT / (D * static_cast<int>(sizeof(T)) / 16);
  __shared__ float s_p[kSplitRows];
  __shared__ float s_ds[kSplitRows];
  __shared__ float s_red[KG * D];
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x / a.splits;
  const int sp = blockIdx.x % a.splits;
  const int N = a.N;
  const int j0 = sp * kSplitRows;
  const int j1 = min(N, j0 + kSplitRows);
  const int n = j1 - j0;
  constexpr int es = sizeof(T);
  const char* qs = lrow(a.q, a.lq, slab, a.H, es, 0);
  const char* ds = lrow(a.dout, a.ldo, slab, a.H, es, 0);
  const size_t rq = a.lq.row_bytes(es), rd = a.ldo.row_bytes(es);
  uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
  frag_load_cached<T, D, G>(lrow(a.k, a.lk, slab, a.H, es, 0), tid % G, kf);
  frag_load_cached<T, D, G>(lrow(a.v, a.lv, slab, a.H, es, 0), tid % G, vf);
  for_rows<G, NT>(j0, j1, [&](int i, int r, int part) {
    uint32_t qf[Gm::kWPL], dof[Gm::kWPL];
    frag_load_cached<T, D, G>(qs + static_cast<size_t>(r) * rq, part, qf);
    frag_load_cached<T, D, G>(ds + static_cast<size_t>(r) * rd, part, dof);
    const float lse2 = a.lse[slab * N + r] * kLog2e;
    const float dj = a.ws_d[slab * N + r];
    const float s = group_sum<G>(M::dot(qf, kf)) * a.scale_log2;
    const float dp = group_sum<G>(M::dot(dof, vf));
    const float p = fast_exp2(s - lse2);
    if (part == 0) {
      s_p[i] = p;
      s_ds[i] = p * (dp - dj);
    }
  });
  __syncthreads();
  const float* cv[1] = {s_p};
  const float* ck[1] = {s_ds};
  float sv[1], sk[1];
  rows_wsum<T, D, NT, 1>(ds, rd, j0, n, cv, s_red, sv);
  rows_wsum<T, D, NT, 1>(qs, rq, j0, n, ck, s_red, sk);
  if (tid < D) {
    if (a.splits == 1) {
      lrow_f32(a.dk, a.ldk, slab, a.H)[tid] = sk[0] * a.scale;
      lrow_f32(a.dv, a.ldv, slab, a.H)[tid] = sv[0];
      lrow_f32(a.dq, a.ldq, slab, a.H)[tid] = a.dq0[slab * D + tid];
    } else {
      float* pp = a.part + (slab * a.splits + sp) * (2 * D);
      pp[tid] = sk[0];
      pp[D + tid] = sv[0];
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
  lrow_f32(a.dk, a.ldk, slab, a.H)[tid] = sk * a.scale;
  lrow_f32(a.dv, a.ldv, slab, a.H)[tid] = sv;
  lrow_f32(a.dq, a.ldq, slab, a.H)[tid] = a.dq0[slab * D + tid];
}

ClsArgs make_args(const Problem& p) {
  ClsArgs a{};
  a.H = p.H;
  a.N = p.N;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.ldo = p.ldo;
  a.ldq = p.ldq;
  a.ldk = p.ldk;
  a.ldv = p.ldv;
  a.splits = cls_splits(p);
  a.scale = 1.0f / sqrtf(static_cast<float>(p.D));
  a.scale_log2 = kLog2e * a.scale;
  return a;
}

template <typename T, int D>
hipError_t fwd_row_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  launch((fwd_cls_row_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    launch((fwd_cls_combine_kernel<T, D>), dim3(slabs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_row_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  launch((bwd_cls_row_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    launch((bwd_cls_row_combine_kernel<D>), dim3(slabs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_col_t(const Problem& p, ClsArgs a, hipStream_t stream) {
  constexpr int G = cls_group<T, D>();
  const unsigned slabs = static_cast<unsigned>(static_cast<size_t>(p.B) * p.H);
  launch((bwd_cls_col_kernel<T, D, G, kClsThreads>), dim3(slabs * a.splits),
                     dim3(kClsThreads), 0, stream, a);
  if (a.splits > 1)
    launch((bwd_cls_col_combine_kernel<D>), dim3(slabs), dim3(D), 0, stream, a);
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

hipError_t launch_fwd_cls(const Problem& p0, const void* q, const void* k, const void* v,
                          void* o, float* lse, float* ws, hipStream_t stream, Path path) {
  Problem p = p0;
  p.cls = true;
  hipError_t e = launch_fwd(p, q, k, v, o, lse, stream, path);
  if (e != hipSuccess) return e;
  // launch_fwd picks the persistent ViT kernel first; that kernel computes
  // the dense row itself when the sequence leaves it a wave without rows.
  if (path == Path::kAuto && fwd_slab_bf16_fits(p) && fwd_slab_bf16_dense_row(p))
    return hipSuccess;
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
  a.dq0 = cls_dq0(p, ws);
  a.part = cls_discard(p, ws) + p.D;
  // The persistent ViT backward kernel computes row 0 and column 0 itself.
  if (path == Path::kAuto && bwd_slab_bf16_fits(p))
    return launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
  // Row 0 first: the key pass of the general kernels needs D_0.
  hipError_t e = bwd_row(p, a, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, ws, stream, path);
  if (e != hipSuccess) return e;
  // Column 0 last: it needs every D_j.
  return bwd_col(p, a, stream);
}

}  // namespace fibatt
