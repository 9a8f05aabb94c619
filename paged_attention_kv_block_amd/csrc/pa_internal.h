// Internal helpers shared by the host and device halves of libpa.
#pragma once

namespace pa {

// Records a printf-style message for pa_last_error() and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// NaN test on the bits, independent of the floating-point build flags.
inline bool is_nan_bits(float x) {
  unsigned u;
  __builtin_memcpy(&u, &x, sizeof u);
  return (u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u;
}

}  // namespace pa
