// Status strings and the per-thread error message of the C entry points.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace ssm {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSM_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return SSM_OK;
}

}  // namespace ssm

extern "C" const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_INVALID_ARG: return "invalid argument";
    case SSM_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSM_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SSM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" const char* ssm_last_error(void) { return ssm::g_last_error; }
