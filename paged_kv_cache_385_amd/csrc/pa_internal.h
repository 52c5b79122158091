// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <cstdarg>
#include <cstdio>

#include "../../include/pa.h"

namespace pa {

// Records a formatted detail for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace pa
