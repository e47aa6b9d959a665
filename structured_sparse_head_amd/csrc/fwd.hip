// Forward kernels: sparse Fibottention attention O = softmax_Omega(Q K^T / sqrt(d)) V.
//
// Fibottention paper (arXiv 2406.19391), method section, eq. (1) and (3):
// only the dot products on the head's support Omega_i are formed; every
// other score is -inf.  The README's Algorithm 3 then applies a row softmax
// and weights V.  Omega_i = {(j, k) : |j - k| in Fib(a_i, b_i), |j - k| <= w_i},
// so for a fixed signed displacement delta the keys k = j + delta of
// consecutive queries j are consecutive rows: a query tile meets, per
// displacement, one contiguous shifted key/value tile.
//
// One lane group (G lanes) owns one query row j and walks the head's signed
// displacements in chunks of C.  Per chunk it forms C scores, rescales its
// running (max, sum, accumulator) once, and accumulates p * V rows: an online
// softmax whose state never leaves registers.  Scores are kept in base 2
// (scaled by log2(e) / sqrt(d)) so the exponentials are single v_exp_f32.
//
// Two variants:
//  * slab: one workgroup per (b, h) slab; the slab's K and V are staged once
//    into LDS with coalesced 16-byte loads (swizzled against bank conflicts)
//    and every shifted tile is read from LDS.  Used when 2*N*d*sizeof(T)
//    fits the LDS budget (e.g. ViT-B/16, N = 197).
//  * stream: one workgroup per query tile; each lane group reads its shifted
//    K/V rows straight from global memory (L2-resident for neighbouring
//    tiles).  Used for long sequences.
#include "kernel_common.h"
#include "launch.h"

namespace fibatt {
namespace {

template <int MH>
struct FwdArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int H;
  int N;
  int tiles;          // query tiles per slab (stream variant)
  float scale_log2;   // log2(e) / sqrt(d)
  Layout lq, lk, lv, lo;
  HeadTableT<MH> ht;
};

template <typename T, int D, int G>
struct LdsKV {
  // Rows come from LDS: reads are unconditional and pipelined (attend_row).
  static constexpr bool kPipelined = true;
  const char* k;
  const char* v;
  __device__ void load_k(int r, int part, uint32_t (&f)[Geom<T, D, G>::kWPL]) const {
    frag_load_lds<T, D, G>(k, r, part, f);
  }
  __device__ void load_v(int r, int part, uint32_t (&f)[Geom<T, D, G>::kWPL]) const {
    frag_load_lds<T, D, G>(v, r, part, f);
  }
};

template <typename T, int D, int G>
struct GlobalKV {
  // Rows come from L2/HBM: only keys in range are read, and latency is left
  // to the other waves (a second register set costs more occupancy than it
  // saves, measured on long fp32 sequences).
  static constexpr bool kPipelined = false;
  const char* k;  // slab base
  const char* v;
  size_t rsk, rsv;  // row strides, bytes
  __device__ void load_k(int r, int part, uint32_t (&f)[Geom<T, D, G>::kWPL]) const {
    frag_load_cached<T, D, G>(k + static_cast<size_t>(r) * rsk, part, f);
  }
  __device__ void load_v(int r, int part, uint32_t (&f)[Geom<T, D, G>::kWPL]) const {
    frag_load_cached<T, D, G>(v + static_cast<size_t>(r) * rsv, part, f);
  }
};

// Online softmax over the signed displacements for query row j.
template <typename T, int D, int G, int C, typename KV>
__device__ __forceinline__ void attend_row(const KV& kv, int j, int N, int part, const int* deltas,
                                           int nd, float scale_log2,
                                           const uint32_t (&qf)[Geom<T, D, G>::kWPL],
                                           float (&acc)[Geom<T, D, G>::kDL], float& m, float& l) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  if constexpr (KV::kPipelined) {
    for (int i0 = 0; i0 < nd; i0 += C) {
      // Keys out of range (or past the list) read row j itself and are
      // masked: every read is unconditional, so the compiler can have several
      // in flight instead of waiting out each one under its own lane mask.
      // The chunk's distances are read first (one wait), then its keys.
      float s[C];
      int key[C];
      bool in[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = i0 + c;
        const int kk = j + deltas[i < nd ? i : 0];
        in[c] = (i < nd) && (kk >= 0) && (kk < N);
        key[c] = in[c] ? kk : j;
      }
      uint32_t kf[2][Gm::kWPL];  // key c + 1 is read while key c is scored
      kv.load_k(key[0], part, kf[0]);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c + 1 < C) kv.load_k(key[c + 1], part, kf[(c + 1) & 1]);
        const float sc = group_sum<G>(M::dot(qf, kf[c & 1])) * scale_log2;
        s[c] = in[c] ? sc : -INFINITY;
      }
      float mc = s[0];
#pragma unroll
      for (int c = 1; c < C; ++c) mc = fmaxf(mc, s[c]);
      const float mn = fmaxf(m, mc);
      if (mn == -INFINITY) continue;  // nothing in range yet
      const float alpha = fast_exp2(m - mn);  // 0 when m = -inf
      l *= alpha;
#pragma unroll
      for (int t = 0; t < Gm::kDL; ++t) acc[t] *= alpha;
      uint32_t vf[2][Gm::kWPL];
      kv.load_v(key[0], part, vf[0]);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c + 1 < C) kv.load_v(key[c + 1], part, vf[(c + 1) & 1]);
        const float p = fast_exp2(s[c] - mn);  // 0 for a masked key
        l += p;
        M::axpy(acc, p, vf[c & 1]);
      }
      m = mn;
    }
  } else {
    for (int i0 = 0; i0 < nd; i0 += C) {
      float s[C];
      int key[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = i0 + c;
        const int kk = j + deltas[i < nd ? i : 0];
        const bool ok = (i < nd) && (kk >= 0) && (kk < N);
        key[c] = ok ? kk : -1;
        float sc = -INFINITY;
        if (ok) {
          uint32_t kf[Gm::kWPL];
          kv.load_k(kk, part, kf);
          sc = group_sum<G>(M::dot(qf, kf)) * scale_log2;
        }
        s[c] = sc;
      }
      float mc = s[0];
#pragma unroll
      for (int c = 1; c < C; ++c) mc = fmaxf(mc, s[c]);
      const float mn = fmaxf(m, mc);
      if (mn == -INFINITY) continue;  // nothing in range yet
      const float alpha = fast_exp2(m - mn);  // 0 when m = -inf
      l *= alpha;
#pragma unroll
      for (int t = 0; t < Gm::kDL; ++t) acc[t] *= alpha;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (key[c] >= 0) {
          const float p = fast_exp2(s[c] - mn);
          l += p;
          uint32_t vf[Gm::kWPL];
          kv.load_v(key[c], part, vf);
          M::axpy(acc, p, vf);
        }
      }
      m = mn;
    }
  }
}

// One more key kk for query row j (the class-token column): a single online
// softmax step.
template <typename T, int D, int G, typename KV>
__device__ __forceinline__ void attend_key(const KV& kv, int kk, int part, float scale_log2,
                                           const uint32_t (&qf)[Geom<T, D, G>::kWPL],
                                           float (&acc)[Geom<T, D, G>::kDL], float& m, float& l) {
  using Gm = Geom<T, D, G>;
  using M = FragMath<T, Gm::kWPL>;
  uint32_t kf[Gm::kWPL], vf[Gm::kWPL];
  kv.load_k(kk, part, kf);
  kv.load_v(kk, part, vf);
  const float s = group_sum<G>(M::dot(qf, kf)) * scale_log2;
  const float mn = fmaxf(m, s);
  const float alpha = fast_exp2(m - mn);  // 0 when m = -inf
  const float p = fast_exp2(s - mn);
  l = __builtin_fmaf(l, alpha, p);
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) acc[t] *= alpha;
  M::axpy(acc, p, vf);
  m = mn;
}

// Normalise and write O (in T) and LSE (natural log) for row j.
template <typename T, int D, int G, typename Args>
__device__ __forceinline__ void finish_row(const Args& a, size_t slab, int j, int part,
                                           float (&acc)[Geom<T, D, G>::kDL], float m, float l) {
  using Gm = Geom<T, D, G>;
  const bool has = l > 0.f;
  const float inv = has ? 1.0f / l : 0.f;
  constexpr int es = static_cast<int>(sizeof(T));
  u32x4* orow = reinterpret_cast<u32x4*>(a.o + a.lo.slab_bytes(slab, a.H, es) + j * a.lo.row_bytes(es)) +
                part;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int t = 0; t < Gm::kCPL; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 8 * t + 2 * u;
        w[u] = f32_to_bf16(acc[e] * inv) | (f32_to_bf16(acc[e + 1] * inv) << 16);
      }
      orow[t * G] = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
#pragma unroll
    for (int t = 0; t < Gm::kCPL; ++t) {
      orow[t * G] = u32x4{__float_as_uint(acc[4 * t + 0] * inv), __float_as_uint(acc[4 * t + 1] * inv),
                      __float_as_uint(acc[4 * t + 2] * inv), __float_as_uint(acc[4 * t + 3] * inv)};
    }
  }
  if (part == 0) a.lse[slab * a.N + j] = has ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

// CLS: class-token mask.  Row 0 is left to the dense class-token kernel;
// a row j >= 1 whose distance j to token 0 is not a head distance also
// attends key 0.
template <typename T, int D, int G, int NT, int C, int MH, bool CLS>
__global__ void __launch_bounds__(NT) fwd_slab_kernel(FwdArgs<MH> a) {
  using Gm = Geom<T, D, G>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_deltas[kMaxSigned];
  __shared__ int s_dist[kMaxOffsets];
  __shared__ int s_nd;
  const int tid = threadIdx.x;
  const size_t slab = blockIdx.x;
  const int h = static_cast<int>(slab % a.H);
  const int N = a.N;
  if (tid == 0) build_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  constexpr int es = static_cast<int>(sizeof(T));
  char* lds_k = smem;
  char* lds_v = smem + N * Gm::kRowBytes;
  const char* qbase = a.q + a.lq.slab_bytes(slab, a.H, es);
  const size_t rsq = a.lq.row_bytes(es);
  const int part = tid % G;
  // The first row's Q is requested before K and V are staged, so its
  // latency overlaps the staging.
  const int j0 = tid / G;
  uint32_t qf0[Gm::kWPL];
  if (j0 < N) frag_load_global<T, D, G>(qbase + static_cast<size_t>(j0) * rsq, part, qf0);
  stage2_rows_lds<T, D, NT, true>(lds_k, a.k + a.lk.slab_bytes(slab, a.H, es), a.lk.row_bytes(es),
                                  lds_v, a.v + a.lv.slab_bytes(slab, a.H, es), a.lv.row_bytes(es),
                                  N, tid);
  __syncthreads();
  const int nd = s_nd;
  const LdsKV<T, D, G> kv{lds_k, lds_v};
  for (int j = j0; j < N; j += NT / G) {
    if (CLS && j == 0) continue;
    uint32_t qf[Gm::kWPL];
    if (j == j0) {
#pragma unroll
      for (int u = 0; u < Gm::kWPL; ++u) qf[u] = qf0[u];
    } else {
      frag_load_global<T, D, G>(qbase + static_cast<size_t>(j) * rsq, part, qf);
    }
    float acc[Gm::kDL];
#pragma unroll
    for (int t = 0; t < Gm::kDL; ++t) acc[t] = 0.f;
    float m = -INFINITY, l = 0.f;
    attend_row<T, D, G, C>(kv, j, N, part, s_deltas, nd, a.scale_log2, qf, acc, m, l);
    if (CLS && !has_delta(s_deltas, nd, j))
      attend_key<T, D, G>(kv, 0, part, a.scale_log2, qf, acc, m, l);
    finish_row<T, D, G>(a, slab, j, part, acc, m, l);
  }
}

template <typename T, int D, int G, int NT, int C, int MH, bool CLS>
__global__ void __launch_bounds__(NT) fwd_stream_kernel(FwdArgs<MH> a) {
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
  constexpr int es = static_cast<int>(sizeof(T));
  const GlobalKV<T, D, G> kv{a.k + a.lk.slab_bytes(slab, a.H, es),
                             a.v + a.lv.slab_bytes(slab, a.H, es), a.lk.row_bytes(es),
                             a.lv.row_bytes(es)};
  uint32_t qf[Gm::kWPL];
  frag_load_global<T, D, G>(a.q + a.lq.slab_bytes(slab, a.H, es) + j * a.lq.row_bytes(es), part,
                            qf);
  float acc[Gm::kDL];
#pragma unroll
  for (int t = 0; t < Gm::kDL; ++t) acc[t] = 0.f;
  float m = -INFINITY, l = 0.f;
  attend_row<T, D, G, C>(kv, j, N, part, s_deltas, s_nd, a.scale_log2, qf, acc, m, l);
  if (CLS && !has_delta(s_deltas, s_nd, j))
    attend_key<T, D, G>(kv, 0, part, a.scale_log2, qf, acc, m, l);
  finish_row<T, D, G>(a, slab, j, part, acc, m, l);
}

// Lane-group width per (dtype, d): each lane owns 64 bytes of a row.
template <typename T, int D>
constexpr int fwd_group() {
  return (D * static_cast<int>(sizeof(T))) / 64;
}

template <typename T, int D, int MH, bool CLS>
hipError_t launch_fwd_t(const Problem& p, const void* q, const void* k, const void* v, void* o,
                        float* lse, hipStream_t stream, Path path) {
  constexpr int G = fwd_group<T, D>();
  constexpr int NT = 256;
  constexpr int C = 8;
  using Gm = Geom<T, D, G>;
  FwdArgs<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.H = p.H;
  a.N = p.N;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.ht = shrink_heads<MH>(p.heads, p.H);
  const size_t slabs = static_cast<size_t>(p.B) * p.H;
  const bool slab_ok = fwd_slab_fits(p);
  if (path == Path::kSlab || (path == Path::kAuto && slab_ok)) {
    if (!slab_ok) return hipErrorInvalidValue;
    const size_t lds = 2 * static_cast<size_t>(p.N) * Gm::kRowBytes;
    // One workgroup per CU holds a whole slab: 512 threads, so that a
    // ViT-sized slab takes one pass of row groups.
    constexpr int NTS = 512;
    auto kern = fwd_slab_kernel<T, D, G, NTS, C, MH, CLS>;
    // Opt the kernel into the full slab budget once per process.
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        kSlabLdsBudget);
    if (attr != hipSuccess) return attr;
    a.tiles = 1;
    launch(kern, dim3(static_cast<unsigned>(slabs)), dim3(NTS), lds, stream, a);
  } else {
    const int rows = NT / G;
    a.tiles = (p.N + rows - 1) / rows;
    launch((fwd_stream_kernel<T, D, G, NT, C, MH, CLS>),
                       dim3(static_cast<unsigned>(slabs * a.tiles)), dim3(NT), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_fwd_d(const Problem& p, const void* q, const void* k, const void* v, void* o,
                        float* lse, hipStream_t stream, Path path) {
  if (p.cls) {
    if (p.H <= kSmallHeads)
      return launch_fwd_t<T, D, kSmallHeads, true>(p, q, k, v, o, lse, stream, path);
    return launch_fwd_t<T, D, kMaxHeads, true>(p, q, k, v, o, lse, stream, path);
  }
  if (p.H <= kSmallHeads)
    return launch_fwd_t<T, D, kSmallHeads, false>(p, q, k, v, o, lse, stream, path);
  return launch_fwd_t<T, D, kMaxHeads, false>(p, q, k, v, o, lse, stream, path);
}

}  // namespace

bool fwd_slab_fits(const Problem& p) {
  const int esize = p.dtype == DType::kBF16 ? 2 : 4;
  return 2ll * p.N * p.D * esize <= kSlabLdsBudget;
}

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t stream, Path path) {
  if (path == Path::kAuto && fwd_slab_bf16_fits(p))
    return launch_fwd_slab_bf16(p, q, k, v, o, lse, stream);
  if (path == Path::kAuto && fwd_tile_bf16_fits(p))
    return launch_fwd_tile_bf16(p, q, k, v, o, lse, stream);
  if (p.dtype == DType::kBF16) {
    if (p.D == 64) return launch_fwd_d<bf16_t, 64>(p, q, k, v, o, lse, stream, path);
    if (p.D == 128) return launch_fwd_d<bf16_t, 128>(p, q, k, v, o, lse, stream, path);
  } else {
    if (p.D == 64) return launch_fwd_d<float, 64>(p, q, k, v, o, lse, stream, path);
    if (p.D == 128) return launch_fwd_d<float, 128>(p, q, k, v, o, lse, stream, path);
  }
  return hipErrorInvalidValue;
}

}  // namespace fibatt
