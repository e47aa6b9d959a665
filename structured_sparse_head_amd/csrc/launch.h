// Internal interface between the C entry points and the kernel translation
// units.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "kernel_common.h"

namespace fibatt {

// Events bound by fibatt_time_next_call to the next work-enqueuing call on
// this thread: `start` to the start of its first kernel, `stop` to the end
// of its last one.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool armed = false;
  bool started = false;
};
LaunchEvents& launch_events();

// Clears the events when an entry point returns: they belong to one call.
struct LaunchGuard {
  ~LaunchGuard() {
    LaunchEvents& ev = launch_events();
    ev.armed = false;
    ev.started = false;
    ev.start = ev.stop = nullptr;
  }
};

// Every kernel of the library is launched through here: with events armed it
// goes through hipExtLaunchKernelGGL, which records them at the kernel's own
// start and end on the GPU.
template <typename... KArgs, typename... Args>
inline void launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args&&... args) {
  LaunchEvents& ev = launch_events();
  if (ev.armed) {
    hipExtLaunchKernelGGL(kern, grid, block, static_cast<uint32_t>(lds), stream,
                          ev.started ? nullptr : ev.start, ev.stop, 0,
                          std::forward<Args>(args)...);
    ev.started = true;
  } else {
    hipLaunchKernelGGL(kern, grid, block, lds, stream, std::forward<Args>(args)...);
  }
}

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
