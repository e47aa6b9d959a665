// Problem description shared by the host layer (validation, offset tables,
// workspace sizes: plain C++, built without HIP) and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fib_offsets.h"

namespace fibatt {

constexpr int kMaxHeads = 128;
constexpr int kMaxSigned = 2 * kMaxOffsets;

// Per-head sequence parameters handed to every kernel by value.  Kernel
// arguments are copied at every launch, so kernels are instantiated for a
// small table (up to 16 heads, ~200 bytes) and for the full one.
// Two modes: with `table` null, head h's distances are the terms of
// Fib(a[h], b[h]) up to lim[h]; with `table` set (a caller-supplied device
// array of distances), head h's distances are table[a[h] .. a[h] + b[h]),
// ascending, each below N.
template <int MH>
struct HeadTableT {
  int32_t a[MH];
  int32_t b[MH];
  int32_t lim[MH];  // min(w, N - 1)
  const int32_t* table;
};
using HeadTable = HeadTableT<kMaxHeads>;
constexpr int kSmallHeads = 16;

template <int MH>
HeadTableT<MH> shrink_heads(const HeadTable& t, int H) {
  HeadTableT<MH> r{};
  for (int h = 0; h < H && h < MH; ++h) {
    r.a[h] = t.a[h];
    r.b[h] = t.b[h];
    r.lim[h] = t.lim[h];
  }
  r.table = t.table;
  return r;
}

// Where a tensor's rows live: element (b, h, n, e) of a [B, H, N, D] view is
// at sb b + sh h + sn n + e (elements; the D elements of a row contiguous).
// A dense [B, H, N, D] tensor has sb = H N D, sh = N D, sn = D.
struct Layout {
  int64_t sb, sh, sn;
  // Byte offset of row 0 of slab b H + h, and the byte stride of rows.
  FIBATT_HD size_t slab_bytes(size_t slab, int H, int esize) const {
    return (static_cast<size_t>(slab / H) * sb + static_cast<size_t>(slab % H) * sh) * esize;
  }
  FIBATT_HD size_t row_bytes(int esize) const { return static_cast<size_t>(sn) * esize; }
};

enum class DType : int { kF32 = 0, kBF16 = 1 };

struct Problem {
  int B, H, N, D;
  DType dtype;
  // Fibonacci heads: a, b, lim = min(w, N - 1).  Distance-table heads:
  // a = first index, b = count, heads.table = the device copy of the table.
  HeadTable heads;
  const int32_t* host_table = nullptr;  // host copy of the table, or null
  bool cls = false;  // class-token mask: row and column 0 dense
  // Row layouts of the tensors (dense [B, H, N, D] unless `strided`).
  Layout lq, lk, lv, lo, ldo, ldq, ldk, ldv;
  bool strided = false;
  void dense_layouts() {
    const Layout d{static_cast<int64_t>(H) * N * D, static_cast<int64_t>(N) * D, D};
    lq = lk = lv = lo = ldo = ldq = ldk = ldv = d;
    strided = false;
  }
};

// Ascending distances of head h (at most kMaxOffsets are written).
inline int head_distances(const Problem& p, int h, int32_t* out) {
  if (p.host_table) {
    const int n = p.heads.b[h];
    for (int i = 0; i < n && i < kMaxOffsets; ++i) out[i] = p.host_table[p.heads.a[h] + i];
    return n;
  }
  return fib_offsets_gen(p.heads.a[h], p.heads.b[h], p.heads.lim[h], out, kMaxOffsets);
}

// LDS bytes a workgroup of the general slab-resident kernels may use: all
// of gfx950's 160 KiB but the kernels' static arrays (fp32 ViT-B/16 slabs,
// 2 N d_h 4 = 100 KB, fit; with the 80 KiB that allows two workgroups per CU
// they fell back to the streaming kernels).  With one workgroup per CU these
// kernels run 512 threads.
constexpr int kSlabLdsBudget = 159 * 1024;

// Which kernels a problem runs on; exposed so tests can force a variant.
// kAuto picks the fastest variant whose constraints the problem meets.
enum class Path : int { kAuto = 0, kSlab = 1, kStream = 2 };

// Class-token mask: dense rows are reduced in ranges of kSplitRows rows per
// workgroup.  Backward workspace: D per row [B*H*N], the row kernel's dQ_0
// per slab [B*H*D], one discard row [D], then range partials.
constexpr int kSplitRows = 1024;
inline int cls_splits(const Problem& p) { return (p.N + kSplitRows - 1) / kSplitRows; }
inline int64_t fwd_cls_workspace_floats(const Problem& p) {
  const int s = cls_splits(p);
  return s > 1 ? static_cast<int64_t>(p.B) * p.H * s * (p.D + 2) : 0;
}
inline int64_t bwd_cls_workspace_floats(const Problem& p) {
  const int s = cls_splits(p);
  const int64_t slabs = static_cast<int64_t>(p.B) * p.H;
  return slabs * (p.N + p.D) + p.D + (s > 1 ? slabs * s * (2 * p.D + 1) : 0);
}
inline float* cls_dq0(const Problem& p, float* ws) {
  return ws + static_cast<size_t>(p.B) * p.H * p.N;
}
inline float* cls_discard(const Problem& p, float* ws) {
  return cls_dq0(p, ws) + static_cast<size_t>(p.B) * p.H * p.D;
}

}  // namespace fibatt
