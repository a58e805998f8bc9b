// Thread-local error reporting shared by the host and device halves of the library.
#pragma once

#include "svdq.h"

namespace svdq {
// Formats the thread-local text returned by svdq_last_error() and returns `st`.
svdq_status fail(svdq_status st, const char* fmt, ...);
}  // namespace svdq
