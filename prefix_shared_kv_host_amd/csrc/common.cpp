// Error reporting and version string of the C ABI.
#include <cstdlib>
#include <string>

#include "rkv.h"
#include "rkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace rkv {

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

bool debug_mode() {
  static const bool on = [] {
    const char* v = std::getenv("RKV_DEBUG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

}  // namespace rkv

extern "C" const char* rkv_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* rkv_version(void) { return "rkv 0.1 gfx950"; }
