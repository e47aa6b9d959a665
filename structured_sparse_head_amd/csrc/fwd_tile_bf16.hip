// Forward for long sequences, bf16, d_h = 64 or 128: sparse Fibottention attention
// O = softmax_Omega(Q K^T / sqrt(d)) V on query tiles read straight from
// global memory.
//
// Fibottention paper (arXiv 2406.19391), method section, eq. (1) and (3):
// query row j only meets keys j + delta for the head's signed displacements
// delta (+f and -f for every f in Fib(a_i, b_i) within the window, and 0 when
// 0 is a distance).  For a fixed delta the keys of consecutive queries are
// consecutive rows, so each load instruction of a wave (16 query rows, 8 for
// d_h = 128) reads that many consecutive K or V rows: coalesced, and the rows come from L2 because
// the neighbouring tiles of the slab read the same rows for other
// displacements.
//
// Design points:
//  * Lanes.  A lane quad owns 64 elements of a query row (lane p of the quad:
//    8-element groups p and p + 4 of Q, K, V and O), one quad per row for
//    d_h = 64 and two for 128.  A quad then reads or writes 64 contiguous
//    bytes per instruction, which the cache front end serves as one access
//    (with the four lanes of a row 16 lanes apart every lane was an access of
//    its own, and that access rate bounded the kernel).
//  * Work.  A workgroup (4 waves) takes one query tile of 64 or 32 rows.
//    Tiles are numbered slab by slab and dealt to the XCDs in contiguous
//    ranges (workgroup b runs on XCD b mod 8), so the tiles of a slab share
//    an L2.
//  * Two passes instead of an online softmax.  Pass 1 forms every score of
//    the row in groups of four displacements; a transposed reduction over the
//    quad leaves one full score per lane (displacement 4 g + p in lane p), so
//    a lane keeps ceil(n / 4) scores.  The row maximum is one quad max.
//    Pass 2 turns each lane's own scores into probabilities, broadcasts a
//    group's four within the quad and accumulates P V in fp32.
//  * Lanes past the last row repeat row N - 1 and write identical values.
//  * Class-token mask (CLS): a row j >= 1 whose distance j to token 0 is not
//    a head distance also scores key 0; row 0 is replaced afterwards by the
//    dense class-token row kernel.
#include "tile_bf16_common.h"

namespace fibatt {
namespace {

using slab::clamp_row;
using slab::dot_part;
using namespace tile;


template <int MH>
struct TileArgs {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int H;
  int N;
  int tiles;    // query tiles per slab
  int work;     // slabs * tiles
  int per_xcd;  // tile order: see tile_of_block
  int chunk;
  float scale_log2;
  Layout lq, lk, lv, lo;  // row layouts (read only by the STR kernels)
  HeadTableT<MH> ht;
};

// KG: displacement groups of four the kernel holds scores for (at least
// the largest head's count); smaller instantiations keep fewer registers.
// STR: rows follow the layouts (else dense [B, H, N, d_h], constant strides).
template <int MH, int KG, int NQ, bool CLS, bool STR>
__global__ void __launch_bounds__(kTileThreads) fwd_tile_bf16_kernel(TileArgs<MH> a) {
  using G = Geo<NQ>;
  constexpr int kRowB = G::kRowB;
  __shared__ int s_dist[kMaxOffsets];
  __shared__ __attribute__((aligned(16))) int s_deltas[kMaxSigned + 4];
  __shared__ int s_nd;
  const int w = tile_of_block(a.per_xcd, a.chunk, a.tiles);
  if (w < 0 || w >= a.work) return;  // whole workgroup, before any barrier
  const int slab = w / a.tiles;
  const int tile = w - slab * a.tiles;
  const int h = slab % a.H;
  const int tid = threadIdx.x;
  const int N = a.N;
  const int lane = tid & 63;
  const int part = lane & 3;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  const int row = tile * G::kRows + tile_row<NQ>(tid);
  const int half = row_half<NQ>(tid);
  const int rr = row < N ? row : N - 1;
  const size_t base = static_cast<size_t>(slab) * N * kRowB;
  const int lofs = half * 128 + part * 16;  // this lane's bytes in a row
  // Slab starts and row strides (bytes) of the four tensors.
  const size_t rk = STR ? a.lk.row_bytes(2) : kRowB, rv = STR ? a.lv.row_bytes(2) : kRowB;
  const char* kbase = (STR ? a.k + a.lk.slab_bytes(slab, a.H, 2) : a.k + base) + lofs;
  const char* vbase = (STR ? a.v + a.lv.slab_bytes(slab, a.H, 2) : a.v + base) + lofs;

  // The lane's Q row is requested before the displacement list is built, so
  // its latency overlaps it.
  u32x4 qf[2];
  {
    const char* qrow = STR ? a.q + a.lq.slab_bytes(slab, a.H, 2) + rr * a.lq.row_bytes(2)
                           : a.q + base + static_cast<size_t>(rr) * kRowB;
    qf[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow + lofs));
    qf[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow + lofs + 64));
  }
  if (tid == 0) {
    build_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
    for (int i = 0; i < 4; ++i) s_deltas[s_nd + i] = 0;  // a whole last group
  }
  __syncthreads();
  const int nd = s_nd;
  uint32_t qw[8];
  qw[0] = qf[0].x; qw[1] = qf[0].y; qw[2] = qf[0].z; qw[3] = qf[0].w;
  qw[4] = qf[1].x; qw[5] = qf[1].y; qw[6] = qf[1].z; qw[7] = qf[1].w;

  // Pass 1: scores, one per lane and group of four displacements.  The next
  // group's rows are requested before this group's dot products; one
  // fragment variable per group, so guarded loads merge with nothing.
  float s[KG];
  u32x4 kf[KG][4][2];
  auto load_k = [&](int g) {
    const int4 d4 = *reinterpret_cast<const int4*>(&s_deltas[4 * g]);
    const int d[4] = {__builtin_amdgcn_readfirstlane(d4.x), __builtin_amdgcn_readfirstlane(d4.y),
                      __builtin_amdgcn_readfirstlane(d4.z), __builtin_amdgcn_readfirstlane(d4.w)};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_row_q(kbase + static_cast<size_t>(clamp_row(rr + d[j], N)) * rk, kf[g][j]);
  };
  if (0 < nd) load_k(0);
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    s[g] = -INFINITY;
    if (4 * g < nd) {
      if (g + 1 < KG && 4 * (g + 1) < nd) load_k(g + 1);
      float pd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pd[j] = dot_part(qw, kf[g][j]);
      const float t = halves_sum<NQ>(reduce4q(pd, b0, b1));
      const int kk = rr + s_deltas[4 * g + part];
      const bool ok = 4 * g + part < nd && static_cast<unsigned>(kk) < static_cast<unsigned>(N);
      s[g] = ok ? t : -INFINITY;
    }
  }
  float m = s[0];
#pragma unroll
  for (int g = 1; g < KG; ++g) m = fmaxf(m, s[g]);
  m = quad_max4(m);  // both halves of a row hold the same scores
  float sc = -INFINITY;  // class-token column: key 0
  if constexpr (CLS) {
    u32x4 k0f[2];
    load_row_q(kbase, k0f);
    const float t = halves_sum<NQ>(quad_sum4(dot_part(qw, k0f)));
    sc = (rr >= 1 && !has_delta(s_deltas, nd, rr)) ? t : -INFINITY;
    m = fmaxf(m, sc);
  }

  // Pass 2: P = exp(scale (s - m)), P V in fp32.  A row with no key in its
  // support keeps l = 0 and is written as O = 0, LSE = -inf.  A group's four
  // V rows are requested together, a group ahead (slots past the end have
  // P = 0 and read a valid row).
  const bool any = m != -INFINITY;
  const float c = a.scale_log2;
  const float mc = any ? m * c : 0.f;
  float l = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  u32x4 vf[KG][4][2];
  auto load_v = [&](int g) {
    const int4 d4 = *reinterpret_cast<const int4*>(&s_deltas[4 * g]);
    const int d[4] = {__builtin_amdgcn_readfirstlane(d4.x), __builtin_amdgcn_readfirstlane(d4.y),
                      __builtin_amdgcn_readfirstlane(d4.z), __builtin_amdgcn_readfirstlane(d4.w)};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_row_q(vbase + static_cast<size_t>(clamp_row(rr + d[j], N)) * rv, vf[g][j]);
  };
  if (0 < nd) load_v(0);
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    if (4 * g < nd) {
      if (g + 1 < KG && 4 * (g + 1) < nd) load_v(g + 1);
      const float pown = fast_exp2(__builtin_fmaf(s[g], c, -mc));  // 0 for s = -inf
      l += pown;
      float p[4];
      gather4q(pown, p);
#pragma unroll
      for (int j = 0; j < 4; ++j) axpy_bf16(o, p[j], vf[g][j]);
    }
  }
  l = quad_sum4(l);  // (the other half's l is the same)
  if constexpr (CLS) {
    u32x4 v0f[2];
    load_row_q(vbase, v0f);
    const float p = fast_exp2(__builtin_fmaf(sc, c, -mc));  // 0 for sc = -inf
    l += p;
    axpy_bf16(o, p, v0f);
  }
  const float inv = any ? 1.0f / l : 0.f;
  uint32_t ow[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const __bf16 lo = static_cast<__bf16>(o[2 * u] * inv);
    const __bf16 hi = static_cast<__bf16>(o[2 * u + 1] * inv);
    ow[u] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  char* orow = (STR ? a.o + a.lo.slab_bytes(slab, a.H, 2) + rr * a.lo.row_bytes(2)
                    : a.o + base + static_cast<size_t>(rr) * kRowB) + lofs;
  *reinterpret_cast<u32x4*>(orow) = u32x4{ow[0], ow[1], ow[2], ow[3]};
  *reinterpret_cast<u32x4*>(orow + 64) = u32x4{ow[4], ow[5], ow[6], ow[7]};
  if (part == 0 && half == 0)
    a.lse[static_cast<size_t>(slab) * N + rr] = any ? (mc + fast_log2(l)) * kLn2 : -INFINITY;
}

template <int MH, int KG, int NQ, bool CLS>
void launch_kg(const TileArgs<MH>& a, bool strided, unsigned grid, hipStream_t stream) {
  if (strided)
    launch((fwd_tile_bf16_kernel<MH, KG, NQ, CLS, true>), dim3(grid),
                       dim3(kTileThreads), 0, stream, a);
  else
    launch((fwd_tile_bf16_kernel<MH, KG, NQ, CLS, false>), dim3(grid),
                       dim3(kTileThreads), 0, stream, a);
}

template <int MH, int NQ, bool CLS>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v, void* o,
                    float* lse, hipStream_t stream) {
  TileArgs<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.H = p.H;
  a.N = p.N;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(Geo<NQ>::kD));
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.ht = shrink_heads<MH>(p.heads, p.H);
  const long long slabs = static_cast<long long>(p.B) * p.H;
  a.tiles = (p.N + Geo<NQ>::kRows - 1) / Geo<NQ>::kRows;
  const long long work = slabs * a.tiles;
  if (work > 0x7fffffffll - kXcds) return hipErrorInvalidValue;
  a.work = static_cast<int>(work);
  const long long grid_ll =
      tile_grid(slabs, a.tiles, 2ll * p.N * Geo<NQ>::kRowB, a.per_xcd, a.chunk);
  if (grid_ll > 0x7fffffffll) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(grid_ll);
  const int groups = (max_signed(p) + 3) / 4;
  if (groups <= 4)
    launch_kg<MH, 4, NQ, CLS>(a, p.strided, grid, stream);
  else if (groups <= 8)
    launch_kg<MH, 8, NQ, CLS>(a, p.strided, grid, stream);
  else if (groups <= 12)
    launch_kg<MH, 12, NQ, CLS>(a, p.strided, grid, stream);
  else
    launch_kg<MH, (kMaxSigned + 3) / 4, NQ, CLS>(a, p.strided, grid, stream);
  return hipGetLastError();
}

}  // namespace

bool fwd_tile_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && (p.D == 64 || p.D == 128);
}

template <bool CLS>
hipError_t launch_cls(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t stream) {
  if (p.D == 128) {
    if (p.H <= kSmallHeads) return launch_t<kSmallHeads, 2, CLS>(p, q, k, v, o, lse, stream);
    return launch_t<kMaxHeads, 2, CLS>(p, q, k, v, o, lse, stream);
  }
  if (p.H <= kSmallHeads) return launch_t<kSmallHeads, 1, CLS>(p, q, k, v, o, lse, stream);
  return launch_t<kMaxHeads, 1, CLS>(p, q, k, v, o, lse, stream);
}

hipError_t launch_fwd_tile_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  return p.cls ? launch_cls<true>(p, q, k, v, o, lse, stream)
               : launch_cls<false>(p, q, k, v, o, lse, stream);
}

}  // namespace fibatt
