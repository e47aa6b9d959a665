// C entry points of libfibatt that enqueue GPU work: validation (host.cpp)
// and dispatch to the kernels.  Every check runs on the host before anything
// is enqueued; on error nothing is written and the message is kept per thread
// for fibatt_last_error().  The host-only entry points (Wythoff rows,
// windows, offset table, workspace sizes) live in host.cpp.
#include <hip/hip_runtime.h>

#include "../../include/fibatt.h"
#include "launch.h"
#include "validate.h"

using fibatt::host::check_desc;
using fibatt::host::check_layouts;
using fibatt::host::check_ptr;
using fibatt::host::check_table_desc;
using fibatt::host::fail;
using fibatt::host::ok;
using fibatt::host::path_from_env;

namespace fibatt {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace fibatt

extern "C" {

int fibatt_time_next_call(void* start_event, void* stop_event) {
  fibatt::LaunchEvents& ev = fibatt::launch_events();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(FIBATT_E_INVAL, "start_event and stop_event must both be set or both be NULL");
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  ev.armed = stop_event != nullptr;
  ev.started = false;
  return ok();
}

int fibatt_fwd(const fibatt_desc* desc, const void* q, const void* k, const void* v, void* o,
               float* lse, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")))
    return rc;
  const hipError_t e =
      fibatt::launch_fwd(p, q, k, v, o, lse, static_cast<hipStream_t>(stream), path_from_env());
  if (e != hipSuccess) return fail(FIBATT_E_HIP, "fibatt_fwd launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_bwd(const fibatt_desc* desc, const void* q, const void* k, const void* v,
               const float* lse, const void* dout, float* dq, float* dk, float* dv,
               float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")) ||
      (rc = check_ptr(workspace, "workspace")))
    return rc;
  const hipError_t e =
      fibatt::launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, workspace,
                         static_cast<hipStream_t>(stream), path_from_env());
  if (e != hipSuccess) return fail(FIBATT_E_HIP, "fibatt_bwd launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_fwd_cls(const fibatt_desc* desc, const void* q, const void* k, const void* v, void* o,
                   float* lse, float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")))
    return rc;
  if (fibatt::fwd_cls_workspace_floats(p) > 0 && (rc = check_ptr(workspace, "workspace")))
    return rc;
  const hipError_t e = fibatt::launch_fwd_cls(p, q, k, v, o, lse, workspace,
                                              static_cast<hipStream_t>(stream), path_from_env());
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_fwd_cls launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_bwd_cls(const fibatt_desc* desc, const void* q, const void* k, const void* v,
                   const float* lse, const void* dout, float* dq, float* dk, float* dv,
                   float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")) ||
      (rc = check_ptr(workspace, "workspace")))
    return rc;
  const hipError_t e =
      fibatt::launch_bwd_cls(p, q, k, v, lse, dout, dq, dk, dv, workspace,
                             static_cast<hipStream_t>(stream), path_from_env());
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_bwd_cls launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_fwd_table(const fibatt_table_desc* desc, const void* q, const void* k, const void* v,
                     void* o, float* lse, float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_table_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")))
    return rc;
  if (p.cls && fibatt::fwd_cls_workspace_floats(p) > 0 && (rc = check_ptr(workspace, "workspace")))
    return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = p.cls ? fibatt::launch_fwd_cls(p, q, k, v, o, lse, workspace, s,
                                                      path_from_env())
                             : fibatt::launch_fwd(p, q, k, v, o, lse, s, path_from_env());
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_fwd_table launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_bwd_table(const fibatt_table_desc* desc, const void* q, const void* k, const void* v,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_table_desc(desc, &p);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")) ||
      (rc = check_ptr(workspace, "workspace")))
    return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      p.cls ? fibatt::launch_bwd_cls(p, q, k, v, lse, dout, dq, dk, dv, workspace, s,
                                     path_from_env())
            : fibatt::launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, workspace, s, path_from_env());
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_bwd_table launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_fwd_strided(const fibatt_desc* desc, int32_t cls, const fibatt_layouts* layouts,
                       const void* q, const void* k, const void* v, void* o, float* lse,
                       float* workspace, void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (cls != 0 && cls != 1) return fail(FIBATT_E_INVAL, "cls must be 0 or 1");
  if ((rc = check_layouts(layouts, false, &p))) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")))
    return rc;
  if (cls && fibatt::fwd_cls_workspace_floats(p) > 0 && (rc = check_ptr(workspace, "workspace")))
    return rc;
  const fibatt::Path path = path_from_env();
  hipError_t e;
  if (cls) {
    e = fibatt::launch_fwd_cls(p, q, k, v, o, lse, workspace, static_cast<hipStream_t>(stream),
                               path);
  } else {
    e = fibatt::launch_fwd(p, q, k, v, o, lse, static_cast<hipStream_t>(stream), path);
  }
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_fwd_strided launch: %s", hipGetErrorString(e));
  return ok();
}

int fibatt_bwd_strided(const fibatt_desc* desc, int32_t cls, const fibatt_layouts* layouts,
                       const void* q, const void* k, const void* v, const float* lse,
                       const void* dout, float* dq, float* dk, float* dv, float* workspace,
                       void* stream) {
  fibatt::LaunchGuard guard;
  fibatt::Problem p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (cls != 0 && cls != 1) return fail(FIBATT_E_INVAL, "cls must be 0 or 1");
  if ((rc = check_layouts(layouts, true, &p))) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")) ||
      (rc = check_ptr(workspace, "workspace")))
    return rc;
  const fibatt::Path path = path_from_env();
  hipError_t e;
  if (cls) {
    e = fibatt::launch_bwd_cls(p, q, k, v, lse, dout, dq, dk, dv, workspace,
                               static_cast<hipStream_t>(stream), path);
  } else {
    e = fibatt::launch_bwd(p, q, k, v, lse, dout, dq, dk, dv, workspace,
                           static_cast<hipStream_t>(stream), path);
  }
  if (e != hipSuccess)
    return fail(FIBATT_E_HIP, "fibatt_bwd_strided launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
