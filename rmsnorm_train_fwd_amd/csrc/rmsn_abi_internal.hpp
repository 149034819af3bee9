// rmsn_abi_internal.hpp -- shared by the C ABI's translation units
// (rmsn_abi.cpp, rmsn_noalloc.hip). Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>

#include "rmsnorm_train.h"

#define RMSN_API extern "C" __attribute__((visibility("default")))

namespace rmsn {

// The int a C caller passed for an enum parameter. C allows any int there;
// reading it as the C++ enum would be undefined outside the enumerators'
// range, so the entry points read every enum argument through its bytes and
// pass plain ints on (invalid codes are then rejected by value).
template <class E>
inline int enum_code(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  __builtin_memcpy(&v, &e, sizeof v);
  return v;
}

// Supplies the workspace of a backward call on `stream` once validation and
// planning have passed and the plan needs `need` bytes: sets *ws and
// *ws_bytes, or returns the status the call then returns (nothing has been
// enqueued yet).
typedef rmsn_status (*WorkspaceSource)(void* stream, size_t need, void** ws, size_t* ws_bytes);

// The backward of every form (kPlain, kResidual, kGate): validation, plan,
// launches. With ws_source NULL the caller's (ws, ws_bytes) is the workspace;
// otherwise ws_source provides it.
rmsn_status bwd_common(int form, const void* dy, const void* x, const void* e, const void* w,
                       int w_dtype, const float* rstd, int det, const rmsn_layout* L,
                       void* dx, void* dz, void* dw, int dw_dtype, void* ws,
                       size_t ws_bytes, WorkspaceSource ws_source, const rmsn_launch* o,
                       void* stream);

}  // namespace rmsn
