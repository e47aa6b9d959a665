// fibatt_hbm_stream: a measurement aid that moves a pass's HBM bytes with
// nothing else in it (reads of n_src arrays, writes of n_dst arrays), so the
// bandwidth HBM delivers at that read/write mix on this GPU can be set beside
// the attention kernels' achieved bandwidth.  Grid-stride over 16-byte
// units, non-temporal loads; every written unit is the xor of the units read,
// so no load can be dropped.
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
