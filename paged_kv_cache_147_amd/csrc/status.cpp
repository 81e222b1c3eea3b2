// Status text and the per-thread error detail.
#include "status.h"

namespace pkv {

static thread_local std::string g_last_error;

pa_status fail(pa_status code, const std::string& detail) {
  g_last_error = std::string(pa_strerror(code)) + ": " + detail;
  return code;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace pkv

extern "C" const char* pa_strerror(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_E_INVAL: return "invalid argument";
    case PA_E_NOBLOCKS: return "pool exhausted";
    case PA_E_NOSEQ: return "unknown sequence";
    case PA_E_EXISTS: return "sequence exists";
    case PA_E_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* pa_last_error(void) { return pkv::g_last_error.c_str(); }

extern "C" int32_t pa_version(void) { return 1; }
