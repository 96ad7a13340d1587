// Thread-local error messages and the version string.
#include <cstring>

#include "pkv_internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pkv {

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pkv_status ok() { return PKV_OK; }

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_last_error; }
extern "C" const char* pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }
