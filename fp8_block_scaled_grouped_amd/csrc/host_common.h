// Host-side argument checks shared by the libmoe355 entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe355.h"

namespace moe355 {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE355_OK : MOE355_ELAUNCH;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

}  // namespace moe355

#define MOE355_CHECK(cond, code) \
  do {                           \
    if (!(cond)) return (code);  \
  } while (0)
