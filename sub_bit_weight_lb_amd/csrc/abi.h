// Status helpers shared by the C-ABI translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "nq.h"

namespace nq {
// Record `msg` as the calling thread's last error and return `s`.
nq_status set_error(nq_status s, const std::string& msg);
// Map a HIP error to NQ_ERR_OUT_OF_MEMORY / NQ_ERR_HIP, recording its text.
nq_status hip_error(hipError_t e, const char* what);
}  // namespace nq

#define NQ_HIPCHK(expr)                                     \
  do {                                                      \
    hipError_t _e = (expr);                                 \
    if (_e != hipSuccess) return ::nq::hip_error(_e, #expr); \
  } while (0)
