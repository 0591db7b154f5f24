// Shared state of the host-only stand-ins (stubs.cpp) and the validation
// driver (validation_main.cpp).
#pragma once
#include <stdint.h>

namespace stub {
// Addresses below this are fake device pointers; at or above, host memory.
constexpr uintptr_t kHostFloor = 0x10000000;
extern int launches;          // launches since the last reset
extern int64_t n_tok;         // packed rows of the call in progress (set by the driver)
extern int64_t total_chunks;  // chunks of the last decode split
extern int n_cu;
}  // namespace stub
