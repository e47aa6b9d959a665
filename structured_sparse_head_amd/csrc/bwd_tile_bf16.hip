// Backward for long sequences, bf16, d_h = 64 or 128: exact gradients of the
// sparse Fibottention attention on tiles read straight from global memory.
//
// The Fibottention paper (method section, eq. (1) and (3)) defines the
// forward; the backward is its derivative.  With P the support-restricted
// softmax recomputed from the forward's log-sum-exp, dP_jk = dO_j . V_k,
//   D_j   = sum_k P_jk dP_jk,      dS_jk = P_jk (dP_jk - D_j),
//   dQ_j  = sum_k dS_jk K_k / sqrt(d),
//   dK_k  = sum_j dS_jk Q_j / sqrt(d),   dV_k = sum_j P_jk dO_j.
// The support is symmetric (it is defined through |j - k|), so the queries
// that see key k are k + delta for the same signed displacements: dK and dV
// are gathered key by key, every output row has one writer and no atomics.
//
// Two launches on the caller's stream:
//  * dq: per query row, pass 1 forms P and dP for every displacement (a
//    transposed quad reduction leaves one (P, dP) pair per lane and group of
//    four displacements) and D; pass 2 forms the lane's dS, broadcasts a
//    group's four in the quad and accumulates dS K.  D goes to the workspace.
//  * dkdv: per key row and group of four displacements, the queries' Q and dO
//    rows are read once for both the recomputed scores and the accumulation
//    of dV += P dO and dK += dS Q.
// With d_h = 64 and the plain mask (when the slab's byte offsets fit 32
// bits) the query pass runs as bwd_dq_win_kernel: tiles of 256 rows with the
// K and V rows near the tile in an LDS window (window_bf16_common.h).
// For d_h = 64 the accumulations over a group of four displacements use
// v_dot2_f32_bf16 on pairs of them (axpy4_dot2: P and dS rounded to bf16,
// sums in fp32).  d_h = 128 keeps fp32 coefficients: it is bound by its
// vector-memory traffic, where fewer VALU instructions measured slower.
// Lanes past the last row repeat row N - 1 and write identical values.
#include "tile_bf16_common.h"
#include "window_bf16_common.h"

namespace fibatt {
namespace {

using slab::clamp_row;
using slab::dot_part;
using namespace tile;

template <int MH>
struct BwdTileArgs {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* ws;  // D per row
  int H;
  int N;
  int tiles;
  int work;
  int per_xcd;  // tile order: see tile_of_block
  int chunk;
  float c;      // log2(e) / sqrt(d)
  float scale;  // 1 / sqrt(d)
  Layout lq, lk, lv, ldo, ldq, ldk, ldv;  // row layouts (read only by the STR kernels)
  HeadTableT<MH> ht;
};

// Row r of a slab of bf16 tensor x: the layout's address with STR, else the
// dense one (constant stride).
template <bool STR, int kRowB>
__device__ __forceinline__ const char* tile_row_ptr(const char* x, const Layout& l, size_t slab,
                                                    int H, int N, int r) {
  if constexpr (STR) return x + l.slab_bytes(slab, H, 2) + static_cast<size_t>(r) * l.row_bytes(2);
  return x + (slab * static_cast<size_t>(N) + r) * kRowB;
}

// Row r of a slab of an fp32 output with D elements per row.
template <bool STR, int D>
__device__ __forceinline__ float* tile_row_f32(float* x, const Layout& l, size_t slab, int H,
                                               int N, int r) {
  if constexpr (STR)
    return reinterpret_cast<float*>(reinterpret_cast<char*>(x) + l.slab_bytes(slab, H, 4) +
                                    static_cast<size_t>(r) * l.row_bytes(4));
  return x + (slab * static_cast<size_t>(N) + r) * D;
}

// The head's signed displacements in LDS (thread 0 builds them), padded with
// zeros to a whole last group; returns their count after a barrier.
template <int MH>
__device__ __forceinline__ int stage_deltas(const HeadTableT<MH>& ht, int h, int* dist,
                                            int* deltas, int* nd) {
  if (threadIdx.x == 0) {
    build_deltas(ht, h, dist, deltas, nd);
    for (int i = 0; i < 4; ++i) deltas[*nd + i] = 0;
  }
  __syncthreads();
  return *nd;
}

__device__ __forceinline__ void group_deltas(const int* deltas, int g, int (&d)[4]) {
  const int4 d4 = *reinterpret_cast<const int4*>(&deltas[4 * g]);
  d[0] = __builtin_amdgcn_readfirstlane(d4.x);
  d[1] = __builtin_amdgcn_readfirstlane(d4.y);
  d[2] = __builtin_amdgcn_readfirstlane(d4.z);
  d[3] = __builtin_amdgcn_readfirstlane(d4.w);
}

// Stores this lane's 16 fp32 elements (groups p and p + 4 of its 64-element
// half) times `scale`; `row` already points at the half.
__device__ __forceinline__ void store_row_f32(float* row, int part, const float (&x)[16],
                                              float scale) {
  float4* a = reinterpret_cast<float4*>(row + 8 * part);
  float4* b = reinterpret_cast<float4*>(row + 32 + 8 * part);
  a[0] = make_float4(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
  a[1] = make_float4(x[4] * scale, x[5] * scale, x[6] * scale, x[7] * scale);
  b[0] = make_float4(x[8] * scale, x[9] * scale, x[10] * scale, x[11] * scale);
  b[1] = make_float4(x[12] * scale, x[13] * scale, x[14] * scale, x[15] * scale);
}

__device__ __forceinline__ void frag_words(const u32x4 (&f)[2], uint32_t (&w)[8]) {
  w[0] = f[0].x; w[1] = f[0].y; w[2] = f[0].z; w[3] = f[0].w;
  w[4] = f[1].x; w[5] = f[1].y; w[6] = f[1].z; w[7] = f[1].w;
}

// CLS (class-token mask): a row j >= 1 whose distance j to token 0 is not a
// head distance pairs with token 0: as query (one more term of D_j and dQ_j
// here) and as key (one more term of dK_j and dV_j from query 0 in the key
// kernel, with the dense D_0 that the class-token row kernel left in the
// workspace).  Row 0's D is that D_0; its dQ and key 0's dK and dV are
// replaced by the dense class-token kernels afterwards.
template <int MH, int KG, int NQ, bool CLS, bool STR>
__global__ void __launch_bounds__(kTileThreads) bwd_dq_tile_kernel(BwdTileArgs<MH> a) {
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
  const int N = a.N;
  const int lane = threadIdx.x & 63;
  const int part = lane & 3;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  const int row = tile * G::kRows + tile_row<NQ>(threadIdx.x);
  const int half = row_half<NQ>(threadIdx.x);
  const int rr = row < N ? row : N - 1;
  const size_t rbase = static_cast<size_t>(slab) * N;
  const int lofs = half * 128 + part * 16;  // this lane's bytes in a row
  const char* kbase = tile_row_ptr<STR, kRowB>(a.k, a.lk, slab, a.H, N, 0) + lofs;
  const char* vbase = tile_row_ptr<STR, kRowB>(a.v, a.lv, slab, a.H, N, 0) + lofs;
  const size_t rk = STR ? a.lk.row_bytes(2) : kRowB, rv = STR ? a.lv.row_bytes(2) : kRowB;

  // The lane's own rows are requested before the displacement list is
  // built, so their latency overlaps it.
  u32x4 qf[2], df[2];
  load_row_q(tile_row_ptr<STR, kRowB>(a.q, a.lq, slab, a.H, N, rr) + lofs, qf);
  load_row_q(tile_row_ptr<STR, kRowB>(a.dout, a.ldo, slab, a.H, N, rr) + lofs, df);
  const float lse_r = a.lse[rbase + rr];
  const int nd = stage_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  uint32_t qw[8], dw[8];
  frag_words(qf, qw);
  frag_words(df, dw);
  const float lse2 = lse_r * kLog2e;

  if constexpr (NQ == 2) {
    // d_h = 128: one pass.  With A = sum_k P dP K and S = sum_k P K over the
    // row's keys, dQ sqrt(d) = sum_k P (dP - D) K = A - D S, and
    // D = sum_k P dP is complete at the end, so every K row is read once (a
    // second pass re-read each one, which at long sequences misses L2
    // again).  The coefficients stay fp32.
    float acc_a[16], acc_s[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc_a[e] = 0.f;
      acc_s[e] = 0.f;
    }
    float dl = 0.f;
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      if (4 * g < nd) {
        int d[4];
        group_deltas(s_deltas, g, d);
        u32x4 kf[4][2], vf[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t r = static_cast<size_t>(clamp_row(rr + d[j], N));
          load_row_q(kbase + r * rk, kf[j]);
          load_row_q(vbase + r * rv, vf[j]);
        }
        float ps[4], pp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ps[j] = dot_part(qw, kf[j]);
          pp[j] = dot_part(dw, vf[j]);
        }
        const float sc = halves_sum<NQ>(reduce4q(ps, b0, b1));
        const float dp = halves_sum<NQ>(reduce4q(pp, b0, b1));
        const int kk = rr + s_deltas[4 * g + part];
        const bool ok = 4 * g + part < nd && static_cast<unsigned>(kk) < static_cast<unsigned>(N);
        const float p = ok ? fast_exp2(__builtin_fmaf(sc, a.c, -lse2)) : 0.f;
        dl = __builtin_fmaf(p, dp, dl);
        float pg[4], pdg[4];
        gather4q(p, pg);  // 0 in padded slots
        gather4q(p * dp, pdg);
#pragma unroll
        for (int j = 0; j < 4; ++j) axpy2_bf16(acc_a, pdg[j], acc_s, pg[j], kf[j]);
      }
    }
    float dd = quad_sum4(dl);  // both halves of a row hold the same P, dP
    float pq = 0.f, dpq = 0.f;
    u32x4 k0f[2];
    if constexpr (CLS) {
      u32x4 v0f[2];
      load_row_q(kbase, k0f);
      load_row_q(vbase, v0f);
      const float s = halves_sum<NQ>(quad_sum4(dot_part(qw, k0f)));
      dpq = halves_sum<NQ>(quad_sum4(dot_part(dw, v0f)));
      pq = (rr >= 1 && !has_delta(s_deltas, nd, rr)) ? fast_exp2(__builtin_fmaf(s, a.c, -lse2))
                                                    : 0.f;
      dd = rr == 0 ? a.ws[rbase] : __builtin_fmaf(pq, dpq, dd);  // row 0: the dense D_0
    }
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(-dd, acc_s[e], acc_a[e]);
    if constexpr (CLS) axpy_bf16(acc, pq * (dpq - dd), k0f);
    store_row_f32(tile_row_f32<STR, G::kD>(a.dq, a.ldq, slab, a.H, N, rr) + 64 * half, part, acc,
                  a.scale);
    if (part == 0 && half == 0) a.ws[rbase + rr] = dd;
    return;
  }

  // Pass 1: P and dP, one pair per lane and group; D = sum P dP.
  float pw[KG], dpw[KG];
  float dl = 0.f;
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    pw[g] = 0.f;
    dpw[g] = 0.f;
    if (4 * g < nd) {
      int d[4];
      group_deltas(s_deltas, g, d);
      u32x4 kf[4][2], vf[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t r = static_cast<size_t>(clamp_row(rr + d[j], N));
        load_row_q(kbase + r * rk, kf[j]);
        load_row_q(vbase + r * rv, vf[j]);
      }
      float ps[4], pp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ps[j] = dot_part(qw, kf[j]);
        pp[j] = dot_part(dw, vf[j]);
      }
      const float sc = halves_sum<NQ>(reduce4q(ps, b0, b1));
      const float dp = halves_sum<NQ>(reduce4q(pp, b0, b1));
      const int kk = rr + s_deltas[4 * g + part];
      const bool ok = 4 * g + part < nd && static_cast<unsigned>(kk) < static_cast<unsigned>(N);
      const float p = ok ? fast_exp2(__builtin_fmaf(sc, a.c, -lse2)) : 0.f;
      pw[g] = p;
      dpw[g] = dp;
      dl = __builtin_fmaf(p, dp, dl);
    }
  }
  float dd = quad_sum4(dl);  // both halves of a row hold the same P, dP
  float pq = 0.f, dpq = 0.f;
  if constexpr (CLS) {
    u32x4 k0f[2], v0f[2];
    load_row_q(kbase, k0f);
    load_row_q(vbase, v0f);
    const float s = halves_sum<NQ>(quad_sum4(dot_part(qw, k0f)));
    dpq = halves_sum<NQ>(quad_sum4(dot_part(dw, v0f)));
    pq = (rr >= 1 && !has_delta(s_deltas, nd, rr)) ? fast_exp2(__builtin_fmaf(s, a.c, -lse2)) : 0.f;
    dd = rr == 0 ? a.ws[rbase] : __builtin_fmaf(pq, dpq, dd);  // row 0: the dense D_0
  }

  // Pass 2: dQ = sum dS K / sqrt(d).
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    if (4 * g < nd) {
      float ds[4];
      gather4q(pw[g] * (dpw[g] - dd), ds);  // 0 in padded slots (P = 0 there)
      int d[4];
      group_deltas(s_deltas, g, d);
      if constexpr (NQ == 1) {
        u32x4 kf[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          load_row_q(kbase + static_cast<size_t>(clamp_row(rr + d[j], N)) * rk, kf[j]);
        axpy4_dot2(acc, pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), kf);
      } else {
        // d_h = 128 is bound by rows fetched from beyond L2: no reads for
        // the padded slots.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (4 * g + j < nd) {
            u32x4 kf[2];
            load_row_q(kbase + static_cast<size_t>(clamp_row(rr + d[j], N)) * rk, kf);
            axpy_bf16(acc, ds[j], kf);
          }
        }
      }
    }
  }
  if constexpr (CLS) {
    u32x4 k0f[2];
    load_row_q(kbase, k0f);
    axpy_bf16(acc, pq * (dpq - dd), k0f);
  }
  store_row_f32(tile_row_f32<STR, G::kD>(a.dq, a.ldq, slab, a.H, N, rr) + 64 * half, part, acc,
                a.scale);
  if (part == 0 && half == 0) a.ws[rbase + rr] = dd;
}

template <int MH, int NQ, bool CLS, bool STR>
__global__ void __launch_bounds__(kTileThreads) bwd_dkdv_tile_kernel(BwdTileArgs<MH> a) {
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
  const int N = a.N;
  const int lane = threadIdx.x & 63;
  const int part = lane & 3;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  const int row = tile * G::kRows + tile_row<NQ>(threadIdx.x);
  const int half = row_half<NQ>(threadIdx.x);
  const int rr = row < N ? row : N - 1;  // key row
  const size_t rbase = static_cast<size_t>(slab) * N;
  const int lofs = half * 128 + part * 16;  // this lane's bytes in a row
  const char* qbase = tile_row_ptr<STR, kRowB>(a.q, a.lq, slab, a.H, N, 0) + lofs;
  const char* obase = tile_row_ptr<STR, kRowB>(a.dout, a.ldo, slab, a.H, N, 0) + lofs;
  const size_t rq = STR ? a.lq.row_bytes(2) : kRowB, ro = STR ? a.ldo.row_bytes(2) : kRowB;

  // The lane's own rows are requested before the displacement list is
  // built, so their latency overlaps it.
  u32x4 kf0[2], vf0[2];
  load_row_q(tile_row_ptr<STR, kRowB>(a.k, a.lk, slab, a.H, N, rr) + lofs, kf0);
  load_row_q(tile_row_ptr<STR, kRowB>(a.v, a.lv, slab, a.H, N, rr) + lofs, vf0);
  const int nd = stage_deltas(a.ht, h, s_dist, s_deltas, &s_nd);
  uint32_t kw[8], vw[8];
  frag_words(kf0, kw);
  frag_words(vf0, vw);
  float dk[16], dv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int g = 0; 4 * g < nd; ++g) {
    int d[4];
    group_deltas(s_deltas, g, d);
    // This lane's query (slot p of the group) and its LSE and D, requested
    // with the group's rows.
    const int jj = rr + s_deltas[4 * g + part];
    const bool ok = 4 * g + part < nd && static_cast<unsigned>(jj) < static_cast<unsigned>(N);
    const int jc = clamp_row(jj, N);
    const float lse_j = a.lse[rbase + jc];
    const float d_j = a.ws[rbase + jc];
    u32x4 qf[4][2], of[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t r = static_cast<size_t>(clamp_row(rr + d[j], N));
      load_row_q(qbase + r * rq, qf[j]);
      load_row_q(obase + r * ro, of[j]);
    }
    float ps[4], pp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ps[j] = dot_part(kw, qf[j]);
      pp[j] = dot_part(vw, of[j]);
    }
    const float sc = halves_sum<NQ>(reduce4q(ps, b0, b1));
    const float dp = halves_sum<NQ>(reduce4q(pp, b0, b1));
    const float p = ok ? fast_exp2(__builtin_fmaf(sc, a.c, -lse_j * kLog2e)) : 0.f;
    float pg[4], dsg[4];
    gather4q(p, pg);
    gather4q(p * (dp - d_j), dsg);
    if constexpr (NQ == 1) {
      axpy4_dot2(dv, pack_bf16x2(pg[0], pg[1]), pack_bf16x2(pg[2], pg[3]), of);
      axpy4_dot2(dk, pack_bf16x2(dsg[0], dsg[1]), pack_bf16x2(dsg[2], dsg[3]), qf);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        axpy_bf16(dv, pg[j], of[j]);
        axpy_bf16(dk, dsg[j], qf[j]);
      }
    }
  }
  if constexpr (CLS) {
    u32x4 q0f[2], o0f[2];
    load_row_q(qbase, q0f);
    load_row_q(obase, o0f);
    const float s = halves_sum<NQ>(quad_sum4(dot_part(kw, q0f)));
    const float dp = halves_sum<NQ>(quad_sum4(dot_part(vw, o0f)));
    const float p = (rr >= 1 && !has_delta(s_deltas, nd, rr))
                        ? fast_exp2(__builtin_fmaf(s, a.c, -a.lse[rbase] * kLog2e))
                        : 0.f;
    axpy_bf16(dv, p, o0f);
    axpy_bf16(dk, p * (dp - a.ws[rbase]), q0f);
  }
  // dK and dV go through LDS so that each store instruction writes whole
  // rows (64 lanes x 16 bytes of consecutive rows), and the stores are
  // non-temporal: nothing reads them in this pass, and written back through
  // L2 piecewise at each tile's end they overlapped poorly with the other
  // workgroups' reads (backward of B16 H12 N1569 d64: 201.7 -> 194.0 us).
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int kOutRow = G::kD * 4 + 16;  // fp32 row + 16 bytes against bank conflicts
  constexpr int kRowChunks = G::kD * 4 / 16;
  constexpr int kChunks = G::kRows * kRowChunks;  // per tensor
  __shared__ __attribute__((aligned(16))) char s_out[2 * G::kRows * kOutRow];
  const int trow = row - tile * G::kRows;
  store_row_f32(reinterpret_cast<float*>(s_out + trow * kOutRow) + 64 * half, part, dk, a.scale);
  store_row_f32(reinterpret_cast<float*>(s_out + (G::kRows + trow) * kOutRow) + 64 * half, part, dv,
                1.0f);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 2 * kChunks / kTileThreads; ++t) {
    const int c = threadIdx.x + t * kTileThreads;
    const int tensor = c / kChunks;  // 0: dK, 1: dV
    const int cc = c - tensor * kChunks;
    const int r = cc / kRowChunks, ch = cc - r * kRowChunks;
    const int grow = tile * G::kRows + r;
    if (grow < N) {
      float* orow = tensor == 0 ? tile_row_f32<STR, G::kD>(a.dk, a.ldk, slab, a.H, N, grow)
                                : tile_row_f32<STR, G::kD>(a.dv, a.ldv, slab, a.H, N, grow);
      f32x4v* dst = reinterpret_cast<f32x4v*>(orow) + ch;
      const f32x4v x = *reinterpret_cast<const f32x4v*>(s_out + (tensor * G::kRows + r) * kOutRow + ch * 16);
      __builtin_nontemporal_store(x, dst);
    }
  }
}

// d_h = 64 (plain mask, slab offsets within 32 bits): the query pass on tiles
// of win::kT rows with the K and V rows within win::kDn of the tile staged in
// an LDS window (layout and lane order in window_bf16_common.h), the far ones
// read through buffer loads.
template <int MH, int KG, bool STR>
__global__ void __launch_bounds__(win::kThreads) __attribute__((amdgpu_waves_per_eu(win::kWavesPerSimd)))
bwd_dq_win_kernel(BwdTileArgs<MH> a) {
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
  const int qrow = tid >> 2;
  const int la = lane_unit_a(lane);
  const int dlb = lane_unit_b(lane) - la;
  const int t0 = tile * kT;
  const int row = t0 + qrow;
  const int rr = row < N ? row : N - 1;
  const size_t rbase = static_cast<size_t>(slab) * N;
  const int rk = STR ? static_cast<int>(a.lk.row_bytes(2)) : kRowB16;
  const int rv = STR ? static_cast<int>(a.lv.row_bytes(2)) : kRowB16;
  const Rsrc kres = slab_rsrc(tile_row_ptr<STR, kRowB16>(a.k, a.lk, slab, a.H, N, 0), N, rk);
  const Rsrc vres = slab_rsrc(tile_row_ptr<STR, kRowB16>(a.v, a.lv, slab, a.H, N, 0), N, rv);
  const int wa = ((rr - t0 + kDn) << 7) + la;  // window offset of row rr's fragment a
  const int ka = rr * rk + la, va = rr * rv + la;

  // The window, the lane's own Q and dO rows and its LSE are requested
  // before the displacement list is built.
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
  u32x4 qf[2], df[2];
  {
    const char* qp = tile_row_ptr<STR, kRowB16>(a.q, a.lq, slab, a.H, N, rr);
    const char* dp = tile_row_ptr<STR, kRowB16>(a.dout, a.ldo, slab, a.H, N, rr);
    qf[0] = *reinterpret_cast<const u32x4*>(qp + la);
    qf[1] = *reinterpret_cast<const u32x4*>(qp + la + dlb);
    df[0] = *reinterpret_cast<const u32x4*>(dp + la);
    df[1] = *reinterpret_cast<const u32x4*>(dp + la + dlb);
  }
  const float lse_r = a.lse[rbase + rr];
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
  const int gn = __builtin_amdgcn_readfirstlane(s_gn);
  uint32_t qw[8], dw[8];
  frag_words(qf, qw);
  frag_words(df, dw);
  const float lse2 = lse_r * kLog2e;

  auto load_group = [&](int g, const char* wbase, const Rsrc& res, int ga, int rs,
                        u32x4 (&f)[4][2]) {
    int d[4];
    group_deltas(s_deltas, g, d);
    if (g < gn) {
#pragma unroll
      for (int j = 0; j < 4; ++j) read_frag(wbase, wa + (d[j] << 7), dlb, f[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) buf_frag(res, ga + d[j] * rs, dlb, f[j]);
    }
  };

  // Pass 1: P and dP, one pair per lane and group; D = sum P dP.
  float pw[KG], dpw[KG];
  float dl = 0.f;
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    pw[g] = 0.f;
    dpw[g] = 0.f;
    if (4 * g < nd) {
      u32x4 kf[4][2], vf[4][2];
      load_group(g, kwin, kres, ka, rk, kf);
      load_group(g, vwin, vres, va, rv, vf);
      float ps[4], pp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ps[j] = dot_part(qw, kf[j]);
        pp[j] = dot_part(dw, vf[j]);
      }
      const float sc = reduce4q(ps, b0, b1);
      const float dp = reduce4q(pp, b0, b1);
      const int kk = rr + s_deltas[4 * g + part];
      const bool ok = 4 * g + part < nd && static_cast<unsigned>(kk) < static_cast<unsigned>(N);
      const float p = ok ? fast_exp2(__builtin_fmaf(sc, a.c, -lse2)) : 0.f;
      pw[g] = p;
      dpw[g] = dp;
      dl = __builtin_fmaf(p, dp, dl);
    }
  }
  const float dd = quad_sum4(dl);

  // Pass 2: dQ = sum dS K / sqrt(d).
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    if (4 * g < nd) {
      float ds[4];
      gather4q(pw[g] * (dpw[g] - dd), ds);  // 0 in padded slots (P = 0 there)
      u32x4 kf[4][2];
      load_group(g, kwin, kres, ka, rk, kf);
      axpy4_dot2(acc, pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), kf);
    }
  }
  if (row < N) {
    store_frag_f32(reinterpret_cast<char*>(tile_row_f32<STR, 64>(a.dq, a.ldq, slab, a.H, N, rr)),
                   la, dlb, acc, a.scale);
    if (part == 0) a.ws[rbase + rr] = dd;
  }
}

template <int MH, int KG, int NQ, bool CLS>
void launch_dq(const BwdTileArgs<MH>& a, bool strided, unsigned grid, hipStream_t stream) {
  if (strided)
    launch((bwd_dq_tile_kernel<MH, KG, NQ, CLS, true>), dim3(grid),
                       dim3(kTileThreads), 0, stream, a);
  else
    launch((bwd_dq_tile_kernel<MH, KG, NQ, CLS, false>), dim3(grid),
                       dim3(kTileThreads), 0, stream, a);
}

// Arguments shared by every backward kernel of this file, except the tile
// geometry (tiles, work, per_xcd, chunk), which each launch fills in.
template <int MH>
BwdTileArgs<MH> make_args(const Problem& p, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv,
                          float* ws, int d_h) {
  BwdTileArgs<MH> a;
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
  a.scale = 1.0f / sqrtf(static_cast<float>(d_h));
  a.c = kLog2e * a.scale;
  a.lq = p.lq;
  a.lk = p.lk;
  a.lv = p.lv;
  a.ldo = p.ldo;
  a.ldq = p.ldq;
  a.ldk = p.ldk;
  a.ldv = p.ldv;
  a.ht = shrink_heads<MH>(p.heads, p.H);
  return a;
}

// Tiles of `rows` rows over rows of `row_bytes` bytes: fills in the tile
// geometry of `a` and returns the grid, or -1 when the tile count or the grid
// does not fit an int.
template <int MH>
long long set_tiles(const Problem& p, int rows, int row_bytes, BwdTileArgs<MH>& a) {
  const long long slabs = static_cast<long long>(p.B) * p.H;
  a.tiles = (p.N + rows - 1) / rows;
  const long long work = slabs * a.tiles;
  if (work > 0x7fffffffll - kXcds) return -1;
  a.work = static_cast<int>(work);
  const long long grid = tile_grid(slabs, a.tiles, 2ll * p.N * row_bytes, a.per_xcd, a.chunk);
  return grid > 0x7fffffffll ? -1 : grid;
}

// The key pass on tiles (dK, dV), after a query pass has written D.
template <int MH, int NQ, bool CLS>
hipError_t launch_dkdv(const Problem& p, BwdTileArgs<MH> a, hipStream_t stream) {
  const long long grid = set_tiles(p, Geo<NQ>::kRows, Geo<NQ>::kRowB, a);
  if (grid < 0) return hipErrorInvalidValue;
  if (p.strided)
    launch((bwd_dkdv_tile_kernel<MH, NQ, CLS, true>), dim3(static_cast<unsigned>(grid)),
           dim3(kTileThreads), 0, stream, a);
  else
    launch((bwd_dkdv_tile_kernel<MH, NQ, CLS, false>), dim3(static_cast<unsigned>(grid)),
           dim3(kTileThreads), 0, stream, a);
  return hipGetLastError();
}

template <int MH, int NQ, bool CLS>
hipError_t launch_t(const Problem& p, const void* q, const void* k, const void* v,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    float* ws, hipStream_t stream) {
  BwdTileArgs<MH> a = make_args<MH>(p, q, k, v, lse, dout, dq, dk, dv, ws, Geo<NQ>::kD);
  const long long grid_ll = set_tiles(p, Geo<NQ>::kRows, Geo<NQ>::kRowB, a);
  if (grid_ll < 0) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(grid_ll);
  const int groups = (max_signed(p) + 3) / 4;
  if (groups <= 4)
    launch_dq<MH, 4, NQ, CLS>(a, p.strided, grid, stream);
  else if (groups <= 8)
    launch_dq<MH, 8, NQ, CLS>(a, p.strided, grid, stream);
  else if (groups <= 12)
    launch_dq<MH, 12, NQ, CLS>(a, p.strided, grid, stream);
  else
    launch_dq<MH, (kMaxSigned + 3) / 4, NQ, CLS>(a, p.strided, grid, stream);
  return launch_dkdv<MH, NQ, CLS>(p, a, stream);
}

template <int MH, int KG>
hipError_t launch_dq_win(const BwdTileArgs<MH>& a, bool strided, unsigned grid,
                         hipStream_t stream) {
  constexpr size_t kLds = 2 * win::kTensorBytes;
  static const hipError_t attr_s = win::allow_lds(bwd_dq_win_kernel<MH, KG, true>, kLds);
  static const hipError_t attr_d = win::allow_lds(bwd_dq_win_kernel<MH, KG, false>, kLds);
  if ((strided ? attr_s : attr_d) != hipSuccess) return strided ? attr_s : attr_d;
  launch(strided ? bwd_dq_win_kernel<MH, KG, true> : bwd_dq_win_kernel<MH, KG, false>,
         dim3(grid), dim3(win::kThreads), kLds, stream, a);
  return hipSuccess;
}

// The backward for d_h = 64 with the plain mask: the query pass on the
// window kernel, the key pass on tiles.  (A key pass on LDS windows of Q and
// dO measured slower than the tile kernel: more L2 misses and HBM bytes.)
template <int MH>
hipError_t launch_win(const Problem& p, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      float* ws, hipStream_t stream) {
  BwdTileArgs<MH> a = make_args<MH>(p, q, k, v, lse, dout, dq, dk, dv, ws, 64);
  const long long grid_ll = set_tiles(p, win::kT, win::kRowB, a);
  if (grid_ll < 0) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(grid_ll);
  const int groups = (max_signed(p) + 3) / 4;
  hipError_t e;
  if (groups <= 4)
    e = launch_dq_win<MH, 4>(a, p.strided, grid, stream);
  else if (groups <= 8)
    e = launch_dq_win<MH, 8>(a, p.strided, grid, stream);
  else if (groups <= 12)
    e = launch_dq_win<MH, 12>(a, p.strided, grid, stream);
  else
    e = launch_dq_win<MH, (kMaxSigned + 3) / 4>(a, p.strided, grid, stream);
  if (e != hipSuccess) return e;
  return launch_dkdv<MH, 1, false>(p, a, stream);
}

}  // namespace

bool bwd_tile_bf16_fits(const Problem& p) {
  return p.dtype == DType::kBF16 && (p.D == 64 || p.D == 128);
}

template <bool CLS>
hipError_t launch_cls(const Problem& p, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      float* ws, hipStream_t stream) {
  if (p.D == 128) {
    if (p.H <= kSmallHeads)
      return launch_t<kSmallHeads, 2, CLS>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
    return launch_t<kMaxHeads, 2, CLS>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
  }
  if (!CLS && win::fits(p)) {
    if (p.H <= kSmallHeads)
      return launch_win<kSmallHeads>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
    return launch_win<kMaxHeads>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
  }
  if (p.H <= kSmallHeads)
    return launch_t<kSmallHeads, 1, CLS>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
  return launch_t<kMaxHeads, 1, CLS>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
}

hipError_t launch_bwd_tile_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, float* ws, hipStream_t stream) {
  return p.cls ? launch_cls<true>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream)
               : launch_cls<false>(p, q, k, v, lse, dout, dq, dk, dv, ws, stream);
}

}  // namespace fibatt
