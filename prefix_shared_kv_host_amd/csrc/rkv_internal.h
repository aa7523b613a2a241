// Internal helpers shared by the host tree and the device entry points.
#pragma once

#include <string>

namespace rkv {

// Records a message for rkv_last_error() on this thread and returns `code`.
int fail(int code, const std::string& msg);
// Clears the thread's last error (every entry point calls it first).
void clear_error();
// True when the environment variable RKV_DEBUG is set to a non-zero value.
bool debug_mode();

}  // namespace rkv
