// Internal interface between the C entry points and the kernel translation
// units.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_common.h"

namespace fibatt {

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
// token-0 pairs of rows and keys 1..N-1, plus the dense row/column kernels
// (workspace layout in problem.h).
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
