// Status strings, per-thread error text and version for libmxq.
#include <hip/hip_runtime.h>

#include <string>

#include "mxq_internal.h"

namespace mxq {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

mxq_status fail(mxq_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

mxq_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    return fail(MXQ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  }
  return MXQ_OK;
}

}  // namespace mxq

extern "C" const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_EINVAL: return "MXQ_EINVAL: invalid argument";
    case MXQ_EUNSUPPORTED: return "MXQ_EUNSUPPORTED: valid but not implemented";
    case MXQ_EHIP: return "MXQ_EHIP: HIP runtime error";
  }
  return "unknown mxq_status";
}

extern "C" const char* mxq_last_error(void) { return mxq::g_last_error.c_str(); }

extern "C" const char* mxq_version(void) { return "libmxq 0.1 (gfx950)"; }
