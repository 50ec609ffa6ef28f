// Thread-local last-error message of the C ABI.
#include <cstdio>
#include <string>

#include "pa_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }
extern "C" int32_t pa_abi_version(void) { return pa::kAbiVersion; }
