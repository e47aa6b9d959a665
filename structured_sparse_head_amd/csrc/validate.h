// Host layer of libfibatt (host.cpp, plain C++ with no HIP dependency):
// argument validation and the per-thread error message, shared with the
// entry points that launch kernels (abi.hip).  Every check runs on the host
// before anything is enqueued.
#pragma once

#include "../../include/fibatt.h"
#include "problem.h"

namespace fibatt {
namespace host {

// Records a formatted message for fibatt_last_error() and returns `code`.
int fail(int code, const char* fmt, ...);
// Clears the message and returns FIBATT_OK.
int ok();

// Shape, type and head checks; fill p (dense layouts).
int check_desc(const fibatt_desc* d, Problem* p);
int check_table_desc(const fibatt_table_desc* d, Problem* p);
// Non-NULL and 16-byte aligned.
int check_ptr(const void* ptr, const char* name);
// Row layouts of the strided entry points (bwd selects which tensors are
// read or written); sets p->strided unless every layout is the dense one.
int check_layouts(const fibatt_layouts* ls, bool bwd, Problem* p);
// Test hook: FIBATT_PATH=slab|stream forces a kernel variant (default auto).
Path path_from_env();

}  // namespace host
}  // namespace fibatt
