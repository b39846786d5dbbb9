// Library information and host-side error state of libqssm.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.hpp"

namespace qssm {

static thread_local std::string g_last_error;

qssm_status fail(qssm_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

qssm_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QSSM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return QSSM_OK;
}

}  // namespace qssm

extern "C" {

const char* qssm_status_string(qssm_status s) {
  switch (s) {
    case QSSM_OK: return "ok";
    case QSSM_ERR_INVALID_ARG: return "invalid argument";
    case QSSM_ERR_UNSUPPORTED: return "unsupported";
    case QSSM_ERR_WORKSPACE: return "workspace missing or too small";
    case QSSM_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* qssm_last_error(void) { return qssm::g_last_error.c_str(); }

int32_t qssm_version(void) { return QSSM_VERSION; }

size_t qssm_args_size(int32_t kind) {
  switch (kind) {
    case 0: return sizeof(qssm_scan_args);
    case 1: return sizeof(qssm_s4d_args);
    case 2: return sizeof(qssm_ssd_args);
    case 3: return sizeof(qssm_update_args);
    case 4: return sizeof(qssm_gemm_args);
    default: return 0;
  }
}

}  // extern "C"
