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
//
// d_h = 64 runs fwd_win_bf16_kernel instead (when the slab's byte offsets
// fit 32 bits): tiles of 256 rows with the near K and V rows staged in an LDS
// window (window_bf16_common.h), far rows through buffer loads, the groups
// walked in runtime loops and P V accumulated with v_dot2_f32_bf16 on pairs
// of displacements.
#include "window_bf16_common.h"
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
  const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
  uint32_t ow[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    ow[u] = pack_bf16x2(o[2 * u] * inv, o[2 * u + 1] * inv);
  }
  char* orow = (STR ? a.o + a.lo.slab_bytes(slab, a.H, 2) + rr * a.lo.row_bytes(2)
                    : a.o + base + static_cast<size_t>(rr) * kRowB) + lofs;
  *reinterpret_cast<u32x4*>(orow) = u32x4{ow[0], ow[1], ow[2], ow[3]};
  *reinterpret_cast<u32x4*>(orow + 64) = u32x4{ow[4], ow[5], ow[6], ow[7]};
  if (part == 0 && half == 0)
    a.lse[static_cast<size_t>(slab) * N + rr] = any ? (mc + fast_log2(l)) * kLn2 : -INFINITY;
}

// d_h = 64: the same two passes on tiles of win::kT rows, with the K and V rows
// within win::kDn of the tile staged in LDS (layout and lane order in
// window_bf16_common.h) and the far ones read through buffer loads whose
// offsets take one add per row.  P V uses v_dot2_f32_bf16 on pairs of displacements
// (axpy4_dot2).
template <int MH, int KG, bool CLS, bool STR>
__global__ void __launch_bounds__(win::kThreads) __attribute__((amdgpu_waves_per_eu(win::kWavesPerSimd)))
fwd_win_bf16_kernel(TileArgs<MH> a) {
  using namespace win;
  constexpr int kRowB16 = Geo<1>::kRowB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const kwin = smem;
  char* const vwin = smem + kTensorBytes;
  __shared__ int s_dist[kMaxOffsets];
  __shared__ __attribute__((aligned(16))) int s_deltas[kMaxSigned + 4];
  __shared__ int s_nd;
  __shared__ int s_gn;
  const int w = tile_of_block(a.per_xcd, a.chunk, a.tiles);
  if (w < 0 || w >= a.work) return;  // whole workgroup, before any barrier
  const int slab = w / a.tiles;
  const int tile = w - slab * a.tiles;
  const int tid = threadIdx.x;
  const int N = a.N;
  const int lane = tid & 63;
  const int part = lane & 3;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  const int qrow = tid >> 2;  // row of the tile (one quad per row)
  const int la = lane_unit_a(lane);  // byte offsets of the lane's two fragments in a row
  const int dlb = lane_unit_b(lane) - la;
  const int t0 = tile * kT;
  const int rk = STR ? static_cast<int>(a.lk.row_bytes(2)) : kRowB16;
  const int rv = STR ? static_cast<int>(a.lv.row_bytes(2)) : kRowB16;
  const Rsrc kres = slab_rsrc(STR ? a.k + a.lk.slab_bytes(slab, a.H, 2)
                                  : a.k + static_cast<size_t>(slab) * N * kRowB16, N, rk);
  const Rsrc vres = slab_rsrc(STR ? a.v + a.lv.slab_bytes(slab, a.H, 2)
                                  : a.v + static_cast<size_t>(slab) * N * kRowB16, N, rv);
  const float c = a.scale_log2;
  const int row = t0 + qrow;
  const int rr = row < N ? row : N - 1;
  const int xr = rr - t0 + kDn;  // window position of row rr
  const int wa = (xr << 7) + la;  // window byte offset of fragment a of row rr
  const int ka = rr * rk + la;    // buffer offsets of fragment a of row rr
  const int va = rr * rv + la;

  // The window (rows t0 - kDn .. t0 + kT + kDn - 1; rows outside the slab
  // read as zeros and are never used unmasked) and the lane's Q row are
  // requested before the displacement list is built, so their latency
  // overlaps it.
  u32x4 wk[kFill][2], wv[kFill][2];
#pragma unroll
  for (int i = 0; i < kFill; ++i) {
    const int x = qrow + i * kT;
    if (x < kR) {
      const int r = t0 - kDn + x;
      buf_frag(kres, r * rk + la, dlb, wk[i]);
      buf_frag(vres, r * rv + la, dlb, wv[i]);
    }
  }
  u32x4 qf[2];
  {
    const char* qrow_p = STR ? a.q + a.lq.slab_bytes(slab, a.H, 2) + rr * a.lq.row_bytes(2)
                             : a.q + (static_cast<size_t>(slab) * N + rr) * kRowB16;
    qf[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow_p + la));
    qf[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow_p + la + dlb));
  }
  if (tid == 0) {
    build_deltas(a.ht, slab % a.H, s_dist, s_deltas, &s_nd);
    for (int i = 0; i < 4; ++i) s_deltas[s_nd + i] = 0;  // a whole last group
    s_gn = near_groups(s_deltas, s_nd);
  }
#pragma unroll
  for (int i = 0; i < kFill; ++i) {
    const int x = qrow + i * kT;
    if (x < kR) {
      write_frag(kwin, (x << 7) + la, dlb, wk[i]);
      write_frag(vwin, (x << 7) + la, dlb, wv[i]);
    }
  }
  __syncthreads();
  // A wave whose rows all lie past the slab (the last tile) has no more work
  // and no barrier follows.
  if (t0 + 16 * __builtin_amdgcn_readfirstlane(tid >> 6) >= N) return;
  const int nd = __builtin_amdgcn_readfirstlane(s_nd);
  const int gn = __builtin_amdgcn_readfirstlane(s_gn);  // near groups
  const int ng = (nd + 3) >> 2;                          // all groups
  uint32_t qw[8];
  qw[0] = qf[0].x; qw[1] = qf[0].y; qw[2] = qf[0].z; qw[3] = qf[0].w;
  qw[4] = qf[1].x; qw[5] = qf[1].y; qw[6] = qf[1].z; qw[7] = qf[1].w;

  // Groups of four displacements are walked in runtime loops: the near
  // groups (the first gn) read the window; the far ones alternate between
  // two register sets, the next group requested before the current one is
  // used, with the last group peeled, so that every wait covers just the
  // group it needs.  Scores live in s[g] (g is wave-uniform, so the
  // register file is indexed directly).
  auto near_group = [&](int g, const char* wbase, u32x4 (&f)[4][2]) {
    int d[4];
    deltas_of(s_deltas, g, d);
#pragma unroll
    for (int j = 0; j < 4; ++j) read_frag(wbase, wa + (d[j] << 7), dlb, f[j]);
  };
  auto far_group = [&](int g, const Rsrc& res, int ga, int rs, u32x4 (&f)[4][2]) {
    int d[4];
    deltas_of(s_deltas, g, d);
#pragma unroll
    for (int j = 0; j < 4; ++j) buf_frag(res, ga + d[j] * rs, dlb, f[j]);
  };

  // Pass 1: scores, one per lane and group.
  float s[KG];
#pragma unroll
  for (int g = 0; g < KG; ++g) s[g] = -INFINITY;
  float m = -INFINITY;
  auto score = [&](int g, const u32x4 (&f)[4][2]) {
    float pd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pd[j] = dot_part(qw, f[j]);
    const float t = reduce4q(pd, b0, b1);
    const int kk = rr + s_deltas[4 * g + part];
    const bool ok = 4 * g + part < nd && static_cast<unsigned>(kk) < static_cast<unsigned>(N);
    const float sv = ok ? t : -INFINITY;
    s[g] = sv;
    m = fmaxf(m, sv);
  };
  u32x4 fa[4][2], fb[4][2];
  for (int g = 0; g < gn; ++g) {
    near_group(g, kwin, fa);
    score(g, fa);
  }
  {
    int g = gn;
    if (g < ng) far_group(g, kres, ka, rk, fa);
    while (g + 1 < ng) {
      far_group(g + 1, kres, ka, rk, fb);
      score(g, fa);
      ++g;
      if (g + 1 >= ng) break;
      far_group(g + 1, kres, ka, rk, fa);
      score(g, fb);
      ++g;
    }
    if (g < ng) {  // the last group, in fa or fb by parity of its distance from gn
      if (((g - gn) & 1) == 0)
        score(g, fa);
      else
        score(g, fb);
    }
  }
  m = quad_max4(m);
  float sc = -INFINITY;  // class-token column: key 0
  if constexpr (CLS) {
    u32x4 k0f[2];
    buf_frag(kres, la, dlb, k0f);
    const float t = quad_sum4(dot_part(qw, k0f));
    sc = (rr >= 1 && !has_delta(s_deltas, nd, rr)) ? t : -INFINITY;
    m = fmaxf(m, sc);
  }

  // Pass 2: P = exp(scale (s - m)), P V.
  const bool any = m != -INFINITY;
  const float mc = any ? m * c : 0.f;
  float l = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  auto accum = [&](int g, const u32x4 (&f)[4][2]) {
    const float pown = fast_exp2(__builtin_fmaf(s[g], c, -mc));  // 0 for s = -inf
    l += pown;
    float p[4];
    gather4q(pown, p);
    axpy4_dot2(o, pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), f);
  };
  for (int g = 0; g < gn; ++g) {
    near_group(g, vwin, fa);
    accum(g, fa);
  }
  {
    int g = gn;
    if (g < ng) far_group(g, vres, va, rv, fa);
    while (g + 1 < ng) {
      far_group(g + 1, vres, va, rv, fb);
      accum(g, fa);
      ++g;
      if (g + 1 >= ng) break;
      far_group(g + 1, vres, va, rv, fa);
      accum(g, fb);
      ++g;
    }
    if (g < ng) {
      if (((g - gn) & 1) == 0)
        accum(g, fa);
      else
        accum(g, fb);
    }
  }
  l = quad_sum4(l);
  if constexpr (CLS) {
    u32x4 v0f[2];
    buf_frag(vres, la, dlb, v0f);
    const float p = fast_exp2(__builtin_fmaf(sc, c, -mc));  // 0 for sc = -inf
    l += p;
    axpy_bf16(o, p, v0f);
  }
  const float inv = any ? __builtin_amdgcn_rcpf(l) : 0.f;
  uint32_t ow[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) ow[u] = pack_bf16x2(o[2 * u] * inv, o[2 * u + 1] * inv);
  if (row < N) {
    char* orow = STR ? a.o + a.lo.slab_bytes(slab, a.H, 2) + rr * a.lo.row_bytes(2)
                     : a.o + (static_cast<size_t>(slab) * N + rr) * kRowB16;
    *reinterpret_cast<u32x4*>(orow + la) = u32x4{ow[0], ow[1], ow[2], ow[3]};
    *reinterpret_cast<u32x4*>(orow + la + dlb) = u32x4{ow[4], ow[5], ow[6], ow[7]};
    if (part == 0)
      a.lse[static_cast<size_t>(slab) * N + rr] = any ? (mc + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

template <int MH, int KG, int NQ, bool CLS>
void launch_kg(const TileArgs<MH>& a, bool strided, unsigned grid, hipStream_t stream) {
  if (strided)
    launch((fwd_tile_bf16_kernel<MH, KG, NQ, CLS, true>), dim3(grid), dim3(kTileThreads), 0,
           stream, a);
  else
    launch((fwd_tile_bf16_kernel<MH, KG, NQ, CLS, false>), dim3(grid), dim3(kTileThreads), 0,
           stream, a);
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

template <int MH, int KG, bool CLS>
hipError_t launch_win_kg(const TileArgs<MH>& a, bool strided, unsigned grid, hipStream_t stream) {
  constexpr size_t kLds = 2 * win::kTensorBytes;
  // The window takes more than the default 64 KiB of dynamic LDS.
  static const hipError_t attr_s = win::allow_lds(fwd_win_bf16_kernel<MH, KG, CLS, true>, kLds);
  static const hipError_t attr_d = win::allow_lds(fwd_win_bf16_kernel<MH, KG, CLS, false>, kLds);
  if ((strided ? attr_s : attr_d) != hipSuccess) return strided ? attr_s : attr_d;
  auto kern = strided ? fwd_win_bf16_kernel<MH, KG, CLS, true>
                      : fwd_win_bf16_kernel<MH, KG, CLS, false>;
  launch(kern, dim3(grid), dim3(win::kThreads), kLds, stream, a);
  return hipSuccess;
}

template <int MH, bool CLS>
hipError_t launch_win(const Problem& p, const void* q, const void* k, const void* v, void* o,
                       float* lse, hipStream_t stream) {
  TileArgs<MH> a;
  a.q = static_cast<const char*>(q);
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.H = p.H;
  a.N = p.N;
  a.scale_log2 = kLog2e / 8.0f;  // 1 / sqrt(64)
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.lo = p.lo;
  a.ht = shrink_heads<MH>(p.heads, p.H);
  const long long slabs = static_cast<long long>(p.B) * p.H;
  a.tiles = (p.N + win::kT - 1) / win::kT;
  const long long work = slabs * a.tiles;
  if (work > 0x7fffffffll - kXcds) return hipErrorInvalidValue;
  a.work = static_cast<int>(work);
  const long long grid_ll = tile_grid(slabs, a.tiles, 2ll * p.N * win::kRowB, a.per_xcd, a.chunk);
  if (grid_ll > 0x7fffffffll) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(grid_ll);
  const int groups = (max_signed(p) + 3) / 4;
  hipError_t e;
  if (groups <= 4)
    e = launch_win_kg<MH, 4, CLS>(a, p.strided, grid, stream);
  else if (groups <= 8)
    e = launch_win_kg<MH, 8, CLS>(a, p.strided, grid, stream);
  else if (groups <= 12)
    e = launch_win_kg<MH, 12, CLS>(a, p.strided, grid, stream);
  else
    e = launch_win_kg<MH, (kMaxSigned + 3) / 4, CLS>(a, p.strided, grid, stream);
  return e != hipSuccess ? e : hipGetLastError();
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
  if (win::fits(p)) {
    if (p.H <= kSmallHeads) return launch_win<kSmallHeads, CLS>(p, q, k, v, o, lse, stream);
    return launch_win<kMaxHeads, CLS>(p, q, k, v, o, lse, stream);
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
