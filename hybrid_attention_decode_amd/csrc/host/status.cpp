#include "status.h"

#include <cstdio>
#include <string>

namespace had {
namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return HAD_OK;
}

}  // namespace had

extern "C" int had_abi_version(void) { return HAD_ABI_VERSION; }

extern "C" const char* had_last_error(void) { return had::g_last_error.c_str(); }
