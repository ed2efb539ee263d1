// Thread-local error detail shared by the host side of the library.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "segattn.h"

namespace segattn {

// Records a formatted detail for segattn_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the detail (called at the start of every entry point).
void clear_error();

}  // namespace segattn
