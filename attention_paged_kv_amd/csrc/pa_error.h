// pa_error.h -- the library's per-thread error text, shared by the device API and the host planner.
#pragma once

namespace pa {
// Records printf-style text for pa_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...);
// Clears the text (start of every entry point).
void clear_error();
}  // namespace pa
