// fibatt_bwd_noalloc: the backward of fibatt_bwd for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace the backward kernels need
// (D per row for the tile and general kernels) is a fixed array in the
// library's own device memory, one copy per GPU, instead of a caller buffer.
//
// The array's address is looked up once per device, with that device
// current, through hipGetSymbolAddress; host code never hands the array's
// name itself to a kernel (in host code it is only a stand-in for the symbol,
// not a device address).  Nothing here allocates: no hipMalloc, no hipFree.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fibatt.h"
#include "launch.h"
#include "validate.h"

namespace {

constexpr int64_t kScratchFloats = FIBATT_NOALLOC_MAX_ROWS;
constexpr int kMaxDevices = 64;

// Scratch shared by every fibatt_bwd_noalloc call on a GPU (16 MiB).
static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch`, looked up on first use.
hipError_t scratch_on_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

using fibatt::host::check_desc;
using fibatt::host::check_ptr;
using fibatt::host::fail;
using fibatt::host::ok;
using fibatt::host::path_from_env;

extern "C" int fibatt_bwd_noalloc(const fibatt_desc* desc, const void* q, const void* k,
                                  const void* v, const float* lse, const void* dout, float* dq,
                                  float* dk, float* dv, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")))
    return rc;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  if (rows > kScratchFloats)
    return fail(FIBATT_E_RANGE,
                "fibatt_bwd_noalloc: B*H*N = %lld exceeds FIBATT_NOALLOC_MAX_ROWS = %lld; use "
                "fibatt_bwd with a workspace",
                static_cast<long long>(rows), static_cast<long long>(kScratchFloats));
  float* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_bwd_noalloc scratch lookup: %s", hipGetErrorString(e));
  e = fibatt::launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, ws, static_cast<hipStream_t>(stream),
                         path_from_env());
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_bwd_noalloc launch: %s", hipGetErrorString(e));
  return ok();
}
