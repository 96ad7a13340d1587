// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <cstdarg>
#include <cstdio>

#include "pkv.h"

namespace pkv {

// Records a message for pkv_last_error() on this thread and returns `st`.
pkv_status fail(pkv_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

// Returns PKV_OK (the last error message is kept).
pkv_status ok();

// Device address of pinned host memory mapped into the device's address
// space (hipHostMalloc, torch's pin_memory()), nullptr for other memory.
void* mapped_host(void* host);

}  // namespace pkv
