// Device-side stand-ins for the host-only sanitizer build of the C-ABI layer.
#pragma once

#include <stddef.h>

namespace stub {

// a fresh "device" buffer: 256-byte aligned, inside a reservation the host
// can never read or write
void* dev_alloc(size_t bytes);
// launches recorded since the last reset
void reset_launches();
int launches();
// launch-argument checks that failed so far (each also printed to stderr)
int failures();

}  // namespace stub
