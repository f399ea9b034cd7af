// Library-wide entry points: version and error text.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"

namespace specsam {

static thread_local std::string g_last_error;

int set_error(int rc, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return rc;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(SS_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  return SS_OK;
}

}  // namespace specsam

extern "C" int ss_version(void) { return 100; }

extern "C" const char* ss_last_error_string(void) {
  return specsam::g_last_error.c_str();
}
