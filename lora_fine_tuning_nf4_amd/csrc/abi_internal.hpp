// Internal helpers shared by the ABI translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "lnf4.h"

namespace lnf4 {
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);
}  // namespace lnf4
