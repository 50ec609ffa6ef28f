// Host-side helpers shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "../../include/pa.h"

namespace pa {

// Records a printf-style message as this thread's last error and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears this thread's last error and returns PA_OK.
pa_status ok();

constexpr int32_t kAbiVersion = 1;

}  // namespace pa
