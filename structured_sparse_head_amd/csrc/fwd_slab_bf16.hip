// Forward kernel specialised for short bf16 sequences with d_h = 64
// (ViT-scale token counts, N <= 256): one persistent workgroup per CU walks
// a strided list of (b, h) slabs and overlaps the HBM reads of the next slab
// with the arithmetic on the current one.
//
// Same mathematics as the generic kernels (Fibottention paper, method
// section, eq. (1) and (3); README Algorithm 3): scores Q_j . K_k / sqrt(d)
// on the head's support, a row softmax, P V.  Design points:
//
//  * Lanes.  1024 threads (16 waves, four per SIMD so that LDS and
//    arithmetic latency is hidden by other waves); four lanes own a row:
//    lane l of wave w works on row 16 b_w + (l % 16), where b_w is the
//    wave's row block (plan_blocks), and, with
//    p = (l / 16) xor parity((l % 16) / 4) (see slab_bf16_common.h), on the
//    8-element groups p and p + 4.  The four lanes of a row thus cover
//    each 64-byte half of the bf16 output row together, so every store
//    instruction writes whole 64-byte pieces.  LDS rows are kept permuted
//    (each lane's 16 elements contiguous) so a lane reads its fragment with
//    consecutive 16-byte loads.  K rows stay bf16 and V rows are widened to
//    fp32 while staging, so P V needs no conversions.
//  * Softmax.  All scores of a row (at most 12 distances, each signed, plus
//    0, for N <= 256) stay in registers: one pass forms them, the row
//    maximum is taken once, a second pass exponentiates and accumulates P V
//    in fp32.  No rescaling of the accumulator is needed.  Each pass walks
//    the +f and -f displacements separately: for a wave's 16 rows the useful
//    ones are a prefix of the ascending distances in each direction, so the
//    trip counts are wave-uniform and whole-wave misses are skipped.  Reads
//    are branch-free (out-of-range keys use a clamped row and score -inf);
//    key fragments are double-buffered.
//  * Overlap.  While a slab is computed from LDS, each thread already holds
//    chunks of the next slab's Q, K and V in flight in registers; they are
//    committed to LDS after the next barrier (Q too, so that no prefetch
//    register is carried across the loop).
//  * Class-token mask (CLS): a row j >= 1 whose distance j to token 0 is not
//    a head distance scores key 0 as one more key, like the diagonal.  Row 0
//    attends every key: for N <= 240 at least one wave has no rows of its
//    own, and the first such wave computes that dense row from the slab in
//    LDS (the wave that owns row 0 then stores nothing for it); for longer
//    sequences the dense class-token row kernel replaces row 0 afterwards.
#include "slab_bf16_common.h"

namespace fibatt {
namespace {

using namespace slab;

constexpr int kThreadsF = 1024;                                  // 16 waves
constexpr int kRowsF = kThreadsF / 4;                            // 256 rows
constexpr int kChunksF = kRowsF * (kRowBytes / 16) / kThreadsF;  // 2
constexpr int kGroups = (kMaxPos + 3) / 4;                       // distance groups of four

// Per-head record: bytes 0..11 the ascending positive distances, byte 12
// their count, byte 13 whether 0 is a distance.  Built on the host; with at
// most 16 heads the whole table is 256 bytes of kernel arguments.
// With STR the rows of Q, K, V and O follow their layouts (strided views,
// e.g. of a fused QKV projection); without it they are dense [B, H, N, 64].
template <int MH, bool STR>
struct Args {
  static constexpr bool kStrided = STR;
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int H;
  int N;
  int slabs;
  float scale_log2;
  uint64_t blocks;  // row block of wave w in bits 4 w .. 4 w + 3
  Layout lq, lk, lv, lo;
  u32x4 rec[MH];
};

// Byte address of row r of a slab of tensor x (layout l) for either kind
// of arguments.
template <typename A>
__device__ __forceinline__ const char* slab_row(const A& a, const char* x, const Layout& l,
                                                size_t slab, int N, int r) {
  if constexpr (A::kStrided) {
    return x + l.slab_bytes(slab, a.H, 2) + static_cast<size_t>(r) * l.row_bytes(2);
  } else {
    return x + (slab * static_cast<size_t>(N) + r) * kRowBytes;
  }
}

struct Prefetch {
  u32x4 k[kChunksF];
  u32x4 v[kChunksF];
  u32x4 q[kChunksF];
};

// Loads are unconditional (indices clamped into the slab) so that every
// prefetch register is overwritten each time; only the LDS commit is masked.
// With `idle` set (no next slab) every address collapses onto the slab's
// first row, so the loads cost no HBM traffic.
template <typename A>
__device__ __forceinline__ void issue_prefetch(const A& a, int N, size_t slab, int tid, int row,
                                               int part, bool idle, Prefetch& pf) {
  const int last = idle ? 0 : N * (kRowBytes / 16) - 1;
  if constexpr (A::kStrided) {
    const char* ks = slab_row(a, a.k, a.lk, slab, N, 0);
    const char* vs = slab_row(a, a.v, a.lv, slab, N, 0);
    const char* qs = slab_row(a, a.q, a.lq, slab, N, 0);
    const size_t rk = a.lk.row_bytes(2), rv = a.lv.row_bytes(2), rq = a.lq.row_bytes(2);
#pragma unroll
    for (int c = 0; c < kChunksF; ++c) {
      int idx = tid + c * kThreadsF;
      idx = idx < last ? idx : last;
      const int r = idx >> 3, ch = idx & 7;  // row, 16-byte chunk
      pf.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + r * rk) + ch);
      pf.v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + r * rv) + ch);
      pf.q[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qs + r * rq) + ch);
    }
  } else {
    const size_t base = slab * static_cast<size_t>(N) * kRowBytes;
    const u32x4* ks = reinterpret_cast<const u32x4*>(a.k + base);
    const u32x4* vs = reinterpret_cast<const u32x4*>(a.v + base);
    const u32x4* qs = reinterpret_cast<const u32x4*>(a.q + base);
#pragma unroll
    for (int c = 0; c < kChunksF; ++c) {
      int idx = tid + c * kThreadsF;
      idx = idx < last ? idx : last;
      pf.k[c] = __builtin_nontemporal_load(ks + idx);
      pf.v[c] = __builtin_nontemporal_load(vs + idx);
      pf.q[c] = __builtin_nontemporal_load(qs + idx);
    }
  }
}

// Makes the compiler wait here for every prefetch register.
__device__ __forceinline__ void settle(const Prefetch& pf) {
#pragma unroll
  for (int c = 0; c < kChunksF; ++c) asm volatile("" ::"v"(pf.k[c]), "v"(pf.v[c]), "v"(pf.q[c]));
}

// Chunk ch (8 elements) of row r is element group ch: it becomes logical
// chunk 2 (ch % 4) + ch / 4 of the permuted bf16 row (lane part ch % 4); in
// fp32 it takes logical chunks 4 (ch % 4) + 2 (ch / 4) and the next one.
__device__ __forceinline__ void commit_prefetch(char* lds_k, char* lds_v, char* lds_q, int N,
                                                int tid, const Prefetch& pf) {
  const int chunks = N * (kRowBytes / 16);
#pragma unroll
  for (int c = 0; c < kChunksF; ++c) {
    const int idx = tid + c * kThreadsF;
    if (idx < chunks) {
      const int r = idx >> 3;
      const int ch = idx & 7;
      const int kb = b16_chunk(r, 2 * (ch & 3) + (ch >> 2));
      *reinterpret_cast<u32x4*>(lds_k + kb) = pf.k[c];
      *reinterpret_cast<u32x4*>(lds_q + kb) = pf.q[c];
      const u32x4 x = pf.v[c];
      const int vb = f32_chunk(r, 4 * (ch & 3) + 2 * (ch >> 2));
      *reinterpret_cast<u32x4*>(lds_v + vb) =
          u32x4{x.x << 16, x.x & 0xffff0000u, x.y << 16, x.y & 0xffff0000u};
      *reinterpret_cast<u32x4*>(lds_v + (vb + 16)) =
          u32x4{x.z << 16, x.z & 0xffff0000u, x.w << 16, x.w & 0xffff0000u};
    }
  }
}

// Scores for displacements SGN * f_i, i < n (wave-uniform n), four
// distances per group: each lane forms its partial dot products for the
// group's four keys and one transposed reduction leaves the full score of
// distance 4 g + slot in the lane of that slot (slot = (lane / 16) % 4).
// Out-of-range keys and i >= n score -inf.  The next key fragment is
// requested before the current dot product so LDS latency overlaps
// arithmetic.
template <int SGN>
__device__ __forceinline__ void scores_dir(const RowSpan& ks, Dist dist, int n,
                                           int row, int slot, int N, const uint32_t (&qw)[8],
                                           float (&s)[kGroups]) {
  // One fragment variable per distance (not a two-entry ring): a fragment
  // loaded under a condition then merges with nothing, so the compiler
  // needs no register copies at the branch joins.
  u32x4 kf[kMaxPos][2];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) s[g] = -INFINITY;
  if (n > 0) load_bf16_at(ks.at(SGN * dist.at(0) * kBf16Stride), kf[0]);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (4 * g < n) {
      float pd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        pd[j] = 0.f;
        if (i < n) {
          if (i + 1 < n) load_bf16_at(ks.at(SGN * dist.at(i + 1) * kBf16Stride), kf[i + 1]);
          pd[j] = dot_part(qw, kf[i]);
        }
      }
      const float t = reduce4(pd);
      const uint32_t w = g == 0 ? dist.w0 : (g == 1 ? dist.w1 : dist.w2);
      const int k = row + SGN * static_cast<int>(__builtin_amdgcn_ubfe(w, 8 * slot, 8));
      const bool ok = 4 * g + slot < n && static_cast<unsigned>(k) < static_cast<unsigned>(N);
      s[g] = ok ? t : -INFINITY;
    }
  }
}

// P V for displacements SGN * f_i, i < n: each lane turns its own score of
// a group into a probability, then the group's four are gathered to every
// lane of the row.  l collects this lane's own probabilities only.
template <int SGN>
__device__ __forceinline__ void accumulate_dir(const RowSpan& vs, Dist dist, int n, float c,
                                               float mc,
                                               const float (&s)[kGroups], float& l,
                                               float (&o)[16]) {
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (4 * g < n) {
      const float pown = fast_exp2(__builtin_fmaf(s[g], c, -mc));  // 0 for s = -inf
      l += pown;
      float p[4];
      gather4(pown, p);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        if (i < n) {
          u32x4 vf[4];
          load_f32_at(vs.at(SGN * dist.at(i) * kF32Stride), vf);
          axpy_q(o, p[j], vf);
        }
      }
    }
  }
}

// Dense class-token row for one slab (N <= 240), split over up to
// kDenseWaves of the waves without rows: wave i of n takes the key slots
// t = i, i + n, ... (slot l % 16 of the lane takes keys slot + 16 t) with an
// online softmax, with the same lane parts as a row block.  The wave's slots
// are then combined: a common maximum over the 16 slots (lane bits 0..3),
// the sums rescaled to it, and a lane's P V fragment summed over the 16 lanes
// that hold the same part, which are l ^ x for x in the span of 1, 2, 12 and
// 20 (flipping bits 2 and 3 together, or bits 2 and 4, keeps the part).  The
// wave leaves (max, sum, P V) in LDS; after a barrier the first wave merges
// the parts in order and stores row 0 (one wave alone took longer than the
// rows of the other waves).
constexpr int kDenseSlots = 15;
constexpr int kDenseWaves = 3;
constexpr int kDensePart = 2 + 64;  // max, sum, P V row (parts in lane order)

__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ void dense_part(const float scale_log2, int N, int lane, int wi, int nw,
                                           const char* lds_k, const char* lds_v,
                                           const char* lds_q, float* out) {
  const int slot = lane & 15;
  const int part = lane_part(lane);
  uint32_t qw[8];
  {
    u32x4 qf[2];
    load_bf16_q(lds_q + part * 32, 0, qf);
    qw[0] = qf[0].x; qw[1] = qf[0].y; qw[2] = qf[0].z; qw[3] = qf[0].w;
    qw[4] = qf[1].x; qw[5] = qf[1].y; qw[6] = qf[1].z; qw[7] = qf[1].w;
  }
  const float c = scale_log2;
  float m = -INFINITY, l = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
#pragma unroll 1
  for (int t = wi; t < kDenseSlots; t += nw) {  // uniform trip count; keys past N score -inf
    const int k = slot + 16 * t;
    const int kc = clamp_row(k, N);
    u32x4 kf[2];
    load_bf16_q(lds_k + part * 32, kc, kf);
    const float x = dot_q(qw, kf);
    const float sk = k < N ? x : -INFINITY;
    const float mn = fmaxf(m, sk);
    // A slot with no key yet keeps m = -inf: both exponentials would see
    // -inf - (-inf), so they are chosen explicitly.
    const float alpha = mn == -INFINITY ? 1.f : fast_exp2((m - mn) * c);
    const float p = mn == -INFINITY ? 0.f : fast_exp2((sk - mn) * c);  // 0 for sk = -inf
    u32x4 vf[4];
    load_f32_q(lds_v + part * 64, kc, vf);
    l = __builtin_fmaf(l, alpha, p);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] *= alpha;
    axpy_q(o, p, vf);
    m = mn;
  }
  float mw = m;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) mw = fmaxf(mw, wave_xor(mw, x));  // -inf if no key here
  const float sc = m == -INFINITY ? 0.f : fast_exp2((m - mw) * c);
  l *= sc;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) l += wave_xor(l, x);
  constexpr int kSpan[4] = {1, 2, 12, 20};
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] *= sc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] += wave_xor(o[e], kSpan[i]);
  if (slot == 0) {  // lanes 0, 16, 32, 48: parts 0..3 of the row
#pragma unroll
    for (int e = 0; e < 16; ++e) out[2 + 16 * part + e] = o[e];
    if (lane == 0) {
      out[0] = mw;
      out[1] = l;
    }
  }
}

// Merges the nw parts of the dense row in order and stores row 0 and its
// LSE (lanes of slot 0; key 0 is in part 0, so the maximum is finite).
template <typename A>
__device__ __forceinline__ void dense_store(const A& a, int slab, int N, int lane, int nw,
                                            const float* parts, const Prefetch& pf) {
  const int slot = lane & 15;
  const int part = lane_part(lane);
  const float c = a.scale_log2;
  float mm = parts[0];
  for (int i = 1; i < nw; ++i) mm = fmaxf(mm, parts[i * kDensePart]);
  float l = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  for (int i = 0; i < nw; ++i) {
    const float* pi = parts + i * kDensePart;
    const float w = pi[0] == -INFINITY ? 0.f : fast_exp2((pi[0] - mm) * c);
    l = __builtin_fmaf(pi[1], w, l);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = __builtin_fmaf(pi[2 + 16 * part + e], w, o[e]);
  }
  const float inv = __builtin_amdgcn_rcpf(l);
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    w[u] = pack_bf16x2(o[2 * u] * inv, o[2 * u + 1] * inv);
  }
  settle(pf);
  if (slot == 0) {
    u32x4* orow = reinterpret_cast<u32x4*>(const_cast<char*>(slab_row(a, a.o, a.lo, slab, N, 0)));
    orow[part] = u32x4{w[0], w[1], w[2], w[3]};
    orow[part + 4] = u32x4{w[4], w[5], w[6], w[7]};
    if (lane == 0) a.lse[static_cast<size_t>(slab) * N] = (mm * c + fast_log2(l)) * kLn2;
  }
}

// One slab for an active wave (its first row is < N).  Lanes past the last
// row repeat row N - 1 and store the same values, so the stores need no
// branch and the memory wait counter stays exact around the loop.
template <bool CLS, typename A>
__device__ __forceinline__ void attend_slab(const A& a, int slab, int N, int row, int part, int slot,
                                            int r0,
                                            const char* lds_k, const char* lds_v,
                                            const char* lds_q, Prefetch& pf) {
  const u32x4 rec = a.rec[slab % a.H];
  const Dist dist{rec.x, rec.y, rec.z};
  const int npos = static_cast<int>(rec.w & 0xffu);
  const bool has0 = ((rec.w >> 8) & 0xffu) != 0;
  const int rr = row < N ? row : N - 1;
  uint32_t qw[8];
  {
    u32x4 qf[2];
    load_bf16_q(lds_q + part * 32, rr, qf);
    qw[0] = qf[0].x; qw[1] = qf[0].y; qw[2] = qf[0].z; qw[3] = qf[0].w;
    qw[4] = qf[1].x; qw[5] = qf[1].y; qw[6] = qf[1].z; qw[7] = qf[1].w;
  }
  // Displacements +f are useful to this wave while r0 + f < N, and -f
  // while f <= rl; both are prefixes of the ascending distance list.
  const int rl = (r0 + 15 < N ? r0 + 15 : N - 1);
  int n_plus = 0, n_minus = 0;
  for (int i = 0; i < npos; ++i) {
    const int f = dist.at(i);
    n_plus += (r0 + f < N) ? 1 : 0;
    n_minus += (f <= rl) ? 1 : 0;
  }
  // Pass 1: raw scores Q_j . K_k for every signed displacement (one per
  // lane and group of four distances; the diagonal in every lane).
  float sp[kGroups], sm[kGroups];
  {
    const RowSpan ks(lds_k, kBf16Stride, 32, part, rr, N);
    scores_dir<+1>(ks, dist, n_plus, rr, slot, N, qw, sp);
    scores_dir<-1>(ks, dist, n_minus, rr, slot, N, qw, sm);
  }
  float s0 = -INFINITY;
  if (has0) {
    u32x4 kf[2];
    load_bf16_q(lds_k + part * 32, rr, kf);
    s0 = dot_q(qw, kf);
  }
  float sc = -INFINITY;  // class-token column: key 0
  if constexpr (CLS) {
    u32x4 kf[2];
    load_bf16_q(lds_k + part * 32, 0, kf);
    const float t = dot_q(qw, kf);
    sc = (rr >= 1 && !dist.has(rr, npos)) ? t : -INFINITY;
  }
  float m = fmaxf(fmaxf(sp[0], sm[0]), fmaxf(sp[1], sm[1]));
  m = quad_max(fmaxf(m, fmaxf(sp[2], sm[2])));
  m = fmaxf(m, s0);
  if constexpr (CLS) m = fmaxf(m, sc);
  // Pass 2: P = exp(scale (s - m)), accumulate P V in fp32.  A row with no
  // key in its support keeps l = 0 and is written as O = 0, LSE = -inf.
  const bool any = m != -INFINITY;
  const float c = a.scale_log2;
  const float mc = any ? m * c : 0.f;
  float l = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  {
    const RowSpan vs(lds_v, kF32Stride, 64, part, rr, N);
    accumulate_dir<+1>(vs, dist, n_plus, c, mc, sp, l, o);
    accumulate_dir<-1>(vs, dist, n_minus, c, mc, sm, l, o);
  }
  l = quad_sum(l);
  if (has0) {
    u32x4 vf[4];
    load_f32_q(lds_v + part * 64, rr, vf);
    const float p = fast_exp2(__builtin_fmaf(s0, c, -mc));
    l += p;
    axpy_q(o, p, vf);
  }
  if constexpr (CLS) {
    u32x4 vf[4];
    load_f32_q(lds_v + part * 64, 0, vf);
    const float p = fast_exp2(__builtin_fmaf(sc, c, -mc));  // 0 for sc = -inf
    l += p;
    axpy_q(o, p, vf);
  }
  const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    w[u] = pack_bf16x2(o[2 * u] * inv, o[2 * u + 1] * inv);
  }
  const float lse = any ? (mc + fast_log2(l)) * kLn2 : -INFINITY;
  // The next slab's loads complete before any store of this slab, so the
  // commit after the next barrier waits for nothing.
  settle(pf);
  const size_t grow = static_cast<size_t>(slab) * N + rr;
  u32x4* orow = reinterpret_cast<u32x4*>(const_cast<char*>(slab_row(a, a.o, a.lo, slab, N, rr)));
  // With the class-token mask row 0 is the dense wave's (N <= 240).
  if (!(CLS && rr == 0 && N <= 16 * kDenseSlots)) {
    orow[part] = u32x4{w[0], w[1], w[2], w[3]};
    orow[part + 4] = u32x4{w[4], w[5], w[6], w[7]};
    a.lse[grow] = lse;  // the row's four lanes write the same value
  }
}

template <int MH, bool CLS, bool STR>
__global__ void __launch_bounds__(kThreadsF) fwd_slab_bf16_kernel(Args<MH, STR> a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_dense[CLS ? kDenseWaves * kDensePart : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int r0 = 16 * static_cast<int>((a.blocks >> (4 * wave)) & 15u);
  // With the class-token mask and N <= 240 the waves without rows compute
  // the dense row 0, one more barrier per slab merging their parts.
  const bool dense_on = CLS && a.N <= 16 * kDenseSlots;
  const int row0 = r0 + (lane & 15);
  const int part0 = lane_part(lane);
  const int slot0 = quad_slot(lane);

  // The grid never exceeds the slab count.  The first slab's loads are
  // completed before the loop, so the loop's first trip and later trips see
  // the same pending memory operations.
  Prefetch pf;
  int slab = blockIdx.x;
  issue_prefetch(a, a.N, slab, tid, row0, part0, false, pf);
  settle(pf);
  // Waves whose rows all lie past the sequence only help stage the slabs;
  // they run a loop of their own (same barriers) so that the loop of the
  // working waves has no store-free path.
  if (r0 < a.N) {
    for (; slab < a.slabs; slab += gridDim.x) {
      // Opaque per-slab copies of N and of the lane's row and part keep the
      // address arithmetic inside the loop instead of hoisted into registers.
      int N = a.N;
      asm volatile("" : "+s"(N));
      int row = row0, part = part0, slot = slot0;
      asm volatile("" : "+v"(row), "+v"(part), "+v"(slot));
      char* lds_k = smem;
      char* lds_v = smem + N * kBf16Stride;
      char* lds_q = smem + N * (kBf16Stride + kF32Stride);
      __syncthreads();  // the previous slab is no longer read from LDS
      commit_prefetch(lds_k, lds_v, lds_q, N, tid, pf);
      __syncthreads();
      const int next = slab + gridDim.x;
      issue_prefetch(a, N, next < a.slabs ? next : slab, tid, row, part, next >= a.slabs, pf);
      attend_slab<CLS>(a, slab, N, row, part, slot, r0, lds_k, lds_v, lds_q, pf);
      if (dense_on) __syncthreads();  // the dense row's parts are in LDS
    }
  } else {
    // The first waves without rows compute the class-token row (N <= 240).
    const int first = (a.N + 15) / 16;  // row block of the first wave without rows
    const int nw = 16 - first < kDenseWaves ? 16 - first : kDenseWaves;
    const int wi = r0 / 16 - first;      // this wave's index among them
    const bool dense = dense_on && wi < nw;
    for (; slab < a.slabs; slab += gridDim.x) {
      int N = a.N;
      asm volatile("" : "+s"(N));
      __syncthreads();
      commit_prefetch(smem, smem + N * kBf16Stride, smem + N * (kBf16Stride + kF32Stride), N, tid,
                      pf);
      __syncthreads();
      const int next = slab + gridDim.x;
      issue_prefetch(a, N, next < a.slabs ? next : slab, tid, row0, part0, next >= a.slabs, pf);
      if (dense)
        dense_part(a.scale_log2, N, lane, wi, nw, smem, smem + N * kBf16Stride,
                   smem + N * (kBf16Stride + kF32Stride), s_dense + wi * kDensePart);
      if (dense_on) {
        __syncthreads();
        if (dense && wi == 0) dense_store(a, slab, N, lane, nw, s_dense, pf);
      }
    }
  }
}

template <int MH, bool CLS, bool STR>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v, void* o,
                    float* lse, hipStream_t stream) {
  Args<MH, STR> a;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
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
  a.blocks = plan_blocks(p.N, p.H, a.rec);
  const size_t lds = static_cast<size_t>(p.N) * (2 * kBf16Stride + kF32Stride);
  auto kern = fwd_slab_bf16_kernel<MH, CLS, STR>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          kRowsF * (2 * kBf16Stride + kF32Stride));
  if (attr != hipSuccess) return attr;
  const int cus = cu_count();
  const int grid = a.slabs < cus ? a.slabs : cus;
  launch(kern, dim3(grid), dim3(kThreadsF), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_slab_bf16_dense_row(const Problem& p) { return p.N <= 16 * kDenseSlots; }

bool fwd_slab_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && p.D == 64 && p.N <= kRowsF && records_fit(p);
}

hipError_t launch_fwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  if (p.strided) {
    if (p.cls) {
      if (p.H <= kSmallHeads) return launch_t<kSmallHeads, true, true>(p, q, k, v, o, lse, stream);
      return launch_t<kMaxHeads, true, true>(p, q, k, v, o, lse, stream);
    }
    if (p.H <= kSmallHeads) return launch_t<kSmallHeads, false, true>(p, q, k, v, o, lse, stream);
    return launch_t<kMaxHeads, false, true>(p, q, k, v, o, lse, stream);
  }
  if (p.cls) {
    if (p.H <= kSmallHeads) return launch_t<kSmallHeads, true, false>(p, q, k, v, o, lse, stream);
    return launch_t<kMaxHeads, true, false>(p, q, k, v, o, lse, stream);
  }
  if (p.H <= kSmallHeads) return launch_t<kSmallHeads, false, false>(p, q, k, v, o, lse, stream);
  return launch_t<kMaxHeads, false, false>(p, q, k, v, o, lse, stream);
}

}  // namespace fibatt
