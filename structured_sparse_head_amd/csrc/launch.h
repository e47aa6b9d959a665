// Internal interface between the C entry points and the kernel translation
// units.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_common.h"

namespace fibatt {

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

hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t stream, Path path);

hipError_t launch_bwd(const Problem& p, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      float* workspace, hipStream_t stream, Path path);

bool fwd_slab_fits(const Problem& p);

// Persistent forward for bf16, d_h = 64, N <= 256 (the default when it fits).
bool fwd_slab_bf16_fits(const Problem& p);
// Whether that kernel also computes the dense class-token row (N <= 240).
bool fwd_slab_bf16_dense_row(const Problem& p);
hipError_t launch_fwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream);
// Forward for bf16, d_h = 64 and any N, query tiles read from global memory
// (the default for dense tensors when the persistent kernel does not fit).
bool fwd_tile_bf16_fits(const Problem& p);
hipError_t launch_fwd_tile_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream);
bool bwd_slab_fits(const Problem& p);

// Backward for bf16, d_h = 64 and any N on 64-row tiles (two launches; D
// goes through the workspace); the default for dense tensors when the
// persistent kernel does not fit.
bool bwd_tile_bf16_fits(const Problem& p);
hipError_t launch_bwd_tile_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, float* ws, hipStream_t stream);

// Class-token mask (row and column 0 dense): the general kernels with the
// token-0 pairs of rows and keys 1..N-1, plus the dense row/column kernels.
// Dense rows are reduced in ranges of kSplitRows rows per workgroup.
constexpr int kSplitRows = 1024;
int cls_splits(const Problem& p);
// Backward workspace with the class-token mask: D per row [B*H*N], the row
// kernel's dQ_0 per slab [B*H*D], one discard row [D], then range partials.
inline float* cls_dq0(const Problem& p, float* ws) {
  return ws + static_cast<size_t>(p.B) * p.H * p.N;
}
inline float* cls_discard(const Problem& p, float* ws) {
  return cls_dq0(p, ws) + static_cast<size_t>(p.B) * p.H * p.D;
}
int64_t fwd_cls_workspace_floats(const Problem& p);
int64_t bwd_cls_workspace_floats(const Problem& p);
hipError_t launch_fwd_cls(const Problem& p, const void* q, const void* k, const void* v,
                          void* o, float* lse, float* ws, hipStream_t stream, Path path);
hipError_t launch_bwd_cls(const Problem& p, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv,
                          float* ws, hipStream_t stream, Path path);

// Persistent backward for bf16, d_h = 64, N <= 201 (the default when it fits).
bool bwd_slab_bf16_fits(const Problem& p);
hipError_t launch_bwd_slab_bf16(const Problem& p, const void* q, const void* k, const void* v,
                                const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, float* discard, hipStream_t stream);

}  // namespace fibatt
