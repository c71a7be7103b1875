// Host-side launch helpers shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>

#include "anchorkv_internal.hpp"

namespace akv {

#define AKV_CHECK_LAUNCH(name)                                                              \
  do {                                                                                      \
    hipError_t e_ = hipGetLastError();                                                      \
    if (e_ != hipSuccess) return fail(ANCHORKV_E_HIP, "%s: %s", name, hipGetErrorString(e_)); \
  } while (0)

// Raise a kernel's dynamic-LDS limit to `bytes` (once per size increase).  A
// refusal is cleared from HIP's error state and reported as E_SHAPE.
inline int set_dyn_lds(const void* fn, size_t bytes, size_t* done) {
  if (bytes <= *done) return 0;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ANCHORKV_E_SHAPE, "%zu bytes of LDS not available for this shape", bytes);
  }
  *done = bytes;
  return 0;
}

}  // namespace akv
