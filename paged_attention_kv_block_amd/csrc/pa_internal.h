// Internal helpers shared by the host and device halves of libpa.
#pragma once

namespace pa {

// Records a printf-style message for pa_last_error() and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
