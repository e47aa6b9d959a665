// Forward kernel specialised for short bf16 sequences with d_h = 64
// (ViT-scale token counts, N <= 256): one persistent workgroup per CU walks
// a strided list of (b, h) slabs and overlaps the HBM reads of the next slab
// with the arithmetic on the current one.
//
// Same mathematics as the generic kernels (Fibottention paper, method
// section, eq. (1) and (3); README Algorithm 3): scores Q_j . K_k / sqrt(d)
// on the head's support, a row softmax, P V.  Design points:
//
//  * Lanes and LDS strides as in slab_bf16_common.h.  K rows are kept in
//    bf16 and V rows in fp32 (converted once while staging), so P V needs
//    no conversions.
//  * Softmax.  All scores of a row (at most 12 distances, each signed, plus
//    0, for N <= 256) stay in registers: one pass forms them, the row
//    maximum is taken once, a second pass exponentiates and accumulates P V
//    in fp32.  No rescaling of the accumulator is needed.  Each pass walks
//    the +f and -f displacements separately: for a wave's 32 rows the useful
//    ones are a prefix of the ascending distances in each direction, so the
//    trip counts are wave-uniform and whole-wave misses are skipped.  Reads
//    are branch-free (out-of-range keys use a clamped row and score -inf) and
//    double-buffered so the next fragment is in flight during the arithmetic.
//  * Overlap.  While a slab is computed from LDS, each thread already holds
//    the next slab's K, V chunks and its own Q fragment in flight in
//    registers; they are committed to LDS after the next barrier.
#include "slab_bf16_common.h"

namespace fibatt {
namespace {

using namespace slab;

// Per-head record: bytes 0..11 the ascending positive distances, byte 12
// their count, byte 13 whether 0 is a distance.  Built on the host; with at
// most 16 heads the whole table is 256 bytes of kernel arguments.
template <int MH>
struct Args {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int H;
  int N;
  int slabs;
  float scale_log2;
  u32x4 rec[MH];
};

struct Prefetch {
  u32x4 k[kChunksPerThread];
  u32x4 v[kChunksPerThread];
  u32x4 q[4];
};

// Loads are unconditional (indices clamped into the slab) so that every
// prefetch register is overwritten each time; only the LDS commit is masked.
template <typename A>
__device__ __forceinline__ void issue_prefetch(const A& a, size_t slab, int tid, int row,
                                               int part, Prefetch& pf) {
  const size_t base = slab * static_cast<size_t>(a.N) * kRowBytes;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k + base);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v + base);
  const int last = a.N * (kRowBytes / 16) - 1;
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    int idx = tid + c * kThreads;
    idx = idx < last ? idx : last;
    pf.k[c] = __builtin_nontemporal_load(ks + idx);
    pf.v[c] = __builtin_nontemporal_load(vs + idx);
  }
  const int r = row < a.N ? row : a.N - 1;
  const u32x4* qs =
      reinterpret_cast<const u32x4*>(a.q + base + static_cast<size_t>(r) * kRowBytes + part * 64);
#pragma unroll
  for (int t = 0; t < 4; ++t) pf.q[t] = __builtin_nontemporal_load(qs + t);
}

__device__ __forceinline__ void commit_prefetch(char* lds_k, char* lds_v, int N, int tid,
                                                const Prefetch& pf) {
  const int chunks = N * (kRowBytes / 16);
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    const int idx = tid + c * kThreads;
    if (idx < chunks) {
      const int r = idx >> 3;
      const int ch = idx & 7;
      *reinterpret_cast<u32x4*>(lds_k + r * kBf16Stride + ch * 16) = pf.k[c];
      const u32x4 x = pf.v[c];
      const u32x4 lo = {x.x << 16, x.x & 0xffff0000u, x.y << 16, x.y & 0xffff0000u};
      const u32x4 hi = {x.z << 16, x.z & 0xffff0000u, x.w << 16, x.w & 0xffff0000u};
      *reinterpret_cast<u32x4*>(lds_v + r * kF32Stride + ch * 32) = lo;
      *reinterpret_cast<u32x4*>(lds_v + r * kF32Stride + ch * 32 + 16) = hi;
    }
  }
}


// Scores for displacements sgn * pos[i], i < n (wave-uniform n).  Out-of-range
// keys are read from a clamped row and scored -inf.  The next key fragment is
// requested before the current dot product so LDS latency overlaps arithmetic.
template <int SGN>
__device__ __forceinline__ void scores_dir(const char* lds_k, const int (&pos)[kMaxPos], int n,
                                           int row, int part, int N, const uint32_t (&qw)[16],
                                           float (&s)[kMaxPos]) {
  u32x4 kb[2][4];
  if (n > 0) load_bf16_half(lds_k, clamp_row(row + SGN * pos[0], N), part, kb[0]);
#pragma unroll
  for (int i = 0; i < kMaxPos; ++i) {
    s[i] = -INFINITY;
    if (i < n) {
      if (i + 1 < kMaxPos && i + 1 < n)
        load_bf16_half(lds_k, clamp_row(row + SGN * pos[i + 1 < kMaxPos ? i + 1 : i], N), part,
               kb[(i + 1) & 1]);
      const int kk = row + SGN * pos[i];
      const float d = dot_bf16(qw, kb[i & 1]);
      s[i] = (static_cast<unsigned>(kk) < static_cast<unsigned>(N)) ? d : -INFINITY;
    }
  }
}

template <int SGN>
__device__ __forceinline__ void accumulate_dir(const char* lds_v, const int (&pos)[kMaxPos],
                                               int n, int row, int part, int N, float c, float mc,
                                               const float (&s)[kMaxPos], float& l,
                                               float (&o)[32]) {
  u32x4 vb[2][8];
  if (n > 0) load_f32_half(lds_v, clamp_row(row + SGN * pos[0], N), part, vb[0]);
#pragma unroll
  for (int i = 0; i < kMaxPos; ++i) {
    if (i < n) {
      if (i + 1 < kMaxPos && i + 1 < n)
        load_f32_half(lds_v, clamp_row(row + SGN * pos[i + 1 < kMaxPos ? i + 1 : i], N), part,
               vb[(i + 1) & 1]);
      const float p = fast_exp2(__builtin_fmaf(s[i], c, -mc));  // 0 for s = -inf
      l += p;
      axpy_f32(o, p, vb[i & 1]);
    }
  }
}

template <typename A>
__device__ __forceinline__ void attend_row(const A& a, size_t slab, int row, int part,
                                           const char* lds_k, const char* lds_v,
                                           const int (&pos)[kMaxPos], int n_plus, int n_minus,
                                           bool has0, const u32x4 (&q)[4]) {
  const int N = a.N;
  uint32_t qw[16];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qw[4 * t + 0] = q[t].x;
    qw[4 * t + 1] = q[t].y;
    qw[4 * t + 2] = q[t].z;
    qw[4 * t + 3] = q[t].w;
  }
  // Pass 1: raw scores Q_j . K_k for every signed displacement.
  float sp[kMaxPos], sm[kMaxPos];
  scores_dir<+1>(lds_k, pos, n_plus, row, part, N, qw, sp);
  scores_dir<-1>(lds_k, pos, n_minus, row, part, N, qw, sm);
  float s0 = -INFINITY;
  if (has0) {
    u32x4 kf[4];
    load_bf16_half(lds_k, row, part, kf);
    s0 = dot_bf16(qw, kf);
  }
  float m = s0;
#pragma unroll
  for (int i = 0; i < kMaxPos; ++i) m = fmaxf(m, fmaxf(sp[i], sm[i]));

  const size_t grow = slab * static_cast<size_t>(N) + row;
  u32x4* orow = reinterpret_cast<u32x4*>(a.o + grow * kRowBytes + part * 64);
  if (m == -INFINITY) {  // no key in the support of this row
#pragma unroll
    for (int t = 0; t < 4; ++t) orow[t] = u32x4{0u, 0u, 0u, 0u};
    if (part == 0) a.lse[grow] = -INFINITY;
    return;
  }
  // Pass 2: P = exp(scale (s - m)), accumulate P V in fp32.
  const float c = a.scale_log2;
  const float mc = m * c;
  float l = 0.f;
  float o[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) o[e] = 0.f;
  accumulate_dir<+1>(lds_v, pos, n_plus, row, part, N, c, mc, sp, l, o);
  accumulate_dir<-1>(lds_v, pos, n_minus, row, part, N, c, mc, sm, l, o);
  if (has0) {
    u32x4 vf[8];
    load_f32_half(lds_v, row, part, vf);
    const float p = fast_exp2(__builtin_fmaf(s0, c, -mc));
    l += p;
    axpy_f32(o, p, vf);
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const __bf16 lo = static_cast<__bf16>(o[8 * t + 2 * u] * inv);
      const __bf16 hi = static_cast<__bf16>(o[8 * t + 2 * u + 1] * inv);
      w[u] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    orow[t] = u32x4{w[0], w[1], w[2], w[3]};
  }
  if (part == 0) a.lse[grow] = (mc + fast_log2(l)) * kLn2;
}

template <int MH>
__global__ void __launch_bounds__(kThreads) fwd_slab_bf16_kernel(Args<MH> a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int row = 32 * wave + (lane & 31);
  const int part = lane >> 5;
  const int N = a.N;
  char* lds_k = smem;
  char* lds_v = smem + N * kBf16Stride;
  // Rows of this wave: [32 w, min(32 w + 32, N)).
  const int r0 = 32 * wave;
  const int rl = (r0 + 31 < N ? r0 + 31 : N - 1);

  Prefetch pf;
  int slab = blockIdx.x;
  if (slab < a.slabs) issue_prefetch(a, slab, tid, row, part, pf);
  for (; slab < a.slabs; slab += gridDim.x) {
    __syncthreads();  // the previous slab is no longer read from LDS
    commit_prefetch(lds_k, lds_v, N, tid, pf);
    u32x4 q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) q[t] = pf.q[t];
    __syncthreads();
    const int next = slab + gridDim.x;
    if (next < a.slabs) issue_prefetch(a, next, tid, row, part, pf);
    if (r0 < N) {
      const HeadRecord hr = unpack_record(a.rec[slab % a.H]);
      // Displacements +f are useful to this wave while r0 + f < N, and -f
      // while f <= rl; both are prefixes of the ascending distance list.
      int n_plus = 0, n_minus = 0;
#pragma unroll
      for (int i = 0; i < kMaxPos; ++i) {
        if (i < hr.npos) {
          n_plus += (r0 + hr.pos[i] < N) ? 1 : 0;
          n_minus += (hr.pos[i] <= rl) ? 1 : 0;
        }
      }
      if (row < N)
        attend_row(a, slab, row, part, lds_k, lds_v, hr.pos, n_plus, n_minus, hr.has0, q);
    }
  }
}

template <int MH>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v, void* o,
                    float* lse, hipStream_t stream) {
  Args<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.H = p.H;
  a.N = p.N;
  a.slabs = p.B * p.H;
  a.scale_log2 = kLog2e / 8.0f;  // 1 / sqrt(64)
  if (!pack_records(p, a.rec, MH)) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(p.N) * (kBf16Stride + kF32Stride);
  auto kern = fwd_slab_bf16_kernel<MH>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kMaxRows * (kBf16Stride + kF32Stride));
  if (attr != hipSuccess) return attr;
  const int cus = cu_count();
  const int grid = a.slabs < cus ? a.slabs : cus;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_slab_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && p.D == 64 && p.N <= kMaxRows && records_fit(p);
}

hipError_t launch_fwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  if (p.H <= kSmallHeads) return launch_t<kSmallHeads>(p, q, k, v, o, lse, stream);
  return launch_t<kMaxHeads>(p, q, k, v, o, lse, stream);
}

}  // namespace fibatt
