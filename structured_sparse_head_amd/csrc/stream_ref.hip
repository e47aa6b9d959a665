// Measurement aids.
//
// fibatt_hbm_stream moves a pass's HBM bytes with nothing else in it (reads
// of n_src arrays, writes of n_dst arrays), so the bandwidth HBM delivers at
// that read/write mix on this GPU can be set beside the attention kernels'
// achieved bandwidth.  Grid-stride over 16-byte units, non-temporal loads;
// every written unit is the xor of the units read, so no load can be
// dropped.
//
// fibatt_fabric_read measures the rate at which the XCDs' L2 caches can be
// filled from beyond them (Infinity Cache or HBM): every XCD streams the
// whole buffer, `passes` times, so with a buffer larger than an L2 every
// read misses there.  The long-sequence kernels' L2 misses (their
// FETCH_SIZE) are bounded by this rate.
#include <hip/hip_runtime.h>

#include "../../include/fibatt.h"
#include "launch.h"
#include "validate.h"

namespace {

using fibatt::u32x4;

constexpr int kMaxArrays = 4;
constexpr int kThreads = 256;
constexpr int kBlocks = 4096;

struct StreamArgs {
  const u32x4* src[kMaxArrays];
  u32x4* dst[kMaxArrays];
  int n_src, n_dst, scale;
  int64_t units;  // 16-byte units per source array
};

__global__ void __launch_bounds__(kThreads) hbm_stream_kernel(StreamArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < a.units;
       i += stride) {
    u32x4 x = __builtin_nontemporal_load(a.src[0] + i);
    for (int k = 1; k < a.n_src; ++k) x ^= __builtin_nontemporal_load(a.src[k] + i);
    for (int j = 0; j < a.n_dst; ++j) {
      a.dst[j][i] = x;
      if (a.scale == 2) a.dst[j][a.units + i] = x ^ u32x4{1u, 2u, 3u, 4u};
    }
  }
}

constexpr int kFabricPerXcd = 128;  // workgroups per XCD
constexpr int kFabricUnroll = 8;     // 16-byte units per thread and trip

// Workgroup b runs on XCD b mod 8 (the dispatcher deals workgroups to the
// XCDs round-robin); the kFabricPerXcd workgroups of an XCD stride over all
// `units` of the buffer, `passes` times.  units is a multiple of
// kFabricPerXcd * 256 * kFabricUnroll, so every index is in range.  Each
// workgroup writes the xor of what it read to out[blockIdx.x].
__global__ void __launch_bounds__(kThreads) fabric_read_kernel(const u32x4* __restrict__ a,
                                                               u32x4* __restrict__ out,
                                                               int64_t units, int passes) {
  __shared__ u32x4 red[kThreads];
  const int64_t k = blockIdx.x / 8;
  const int64_t step = static_cast<int64_t>(kFabricPerXcd) * kThreads * kFabricUnroll;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int p = 0; p < passes; ++p) {
    for (int64_t i = k * kThreads * kFabricUnroll + threadIdx.x; i < units; i += step) {
      u32x4 x[kFabricUnroll];
#pragma unroll
      for (int u = 0; u < kFabricUnroll; ++u) x[u] = a[i + u * kThreads];
#pragma unroll
      for (int u = 0; u < kFabricUnroll; ++u) acc ^= x[u];
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w /= 2) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

using fibatt::host::check_ptr;
using fibatt::host::fail;
using fibatt::host::ok;

extern "C" int fibatt_hbm_stream(const void* const* src, int32_t n_src, void* const* dst,
                                 int32_t n_dst, int64_t bytes, int32_t dst_scale, void* stream) {
  fibatt::LaunchGuard guard;
  if (n_src < 1 || n_src > kMaxArrays || n_dst < 1 || n_dst > kMaxArrays)
    return fail(FIBATT_E_INVAL, "fibatt_hbm_stream: 1..4 source and 1..4 destination arrays");
  if (dst_scale != 1 && dst_scale != 2)
    return fail(FIBATT_E_INVAL, "fibatt_hbm_stream: dst_scale must be 1 or 2");
  if (bytes <= 0 || bytes % 16)
    return fail(FIBATT_E_INVAL, "fibatt_hbm_stream: bytes must be a positive multiple of 16");
  if (!src || !dst) return fail(FIBATT_E_INVAL, "fibatt_hbm_stream: NULL array list");
  StreamArgs a{};
  int rc;
  for (int k = 0; k < n_src; ++k) {
    if ((rc = check_ptr(src[k], "src[k]"))) return rc;
    a.src[k] = static_cast<const u32x4*>(src[k]);
  }
  for (int j = 0; j < n_dst; ++j) {
    if ((rc = check_ptr(dst[j], "dst[j]"))) return rc;
    a.dst[j] = static_cast<u32x4*>(dst[j]);
  }
  a.n_src = n_src;
  a.n_dst = n_dst;
  a.scale = dst_scale;
  a.units = bytes / 16;
  const int64_t need = (a.units + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(need < kBlocks ? need : kBlocks);
  fibatt::launch(hbm_stream_kernel, dim3(grid), dim3(kThreads), 0,
                 static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_hbm_stream launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" int fibatt_fabric_read(const void* buf, int64_t bytes, int32_t passes, void* out,
                                  void* stream) {
  fibatt::LaunchGuard guard;
  constexpr int64_t kQuantum =
      static_cast<int64_t>(kFabricPerXcd) * kThreads * kFabricUnroll * 16;  // 4 MiB
  if (bytes <= 0 || bytes % kQuantum)
    return fail(FIBATT_E_INVAL, "fibatt_fabric_read: bytes must be a positive multiple of 4 MiB");
  if (passes < 1) return fail(FIBATT_E_INVAL, "fibatt_fabric_read: passes must be >= 1");
  int rc;
  if ((rc = check_ptr(buf, "buf")) || (rc = check_ptr(out, "out"))) return rc;
  fibatt::launch(fabric_read_kernel, dim3(8 * kFabricPerXcd), dim3(kThreads), 0,
                 static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                 static_cast<u32x4*>(out), bytes / 16, static_cast<int>(passes));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_fabric_read launch: %s", hipGetErrorString(e));
  return ok();
}
