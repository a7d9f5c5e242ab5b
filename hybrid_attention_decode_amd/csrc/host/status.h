// Internal helpers shared by the host-side translation units: thread-local
// error message and status return shortcuts.
#pragma once
#include <cstdarg>
#include <cstdint>

#include "had.h"

namespace had {

// Records a printf-style message for had_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread's last error message and returns HAD_OK.
int ok();

}  // namespace had
