// rmsq_abi_common.h - helpers shared by the library's C-ABI translation units
// (argument checks, the per-thread error message, the device check). Defined
// in rmsq_abi.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsq.h"

namespace rmsq_abi {

// Message of the last error on this thread (rmsq_last_error).
extern thread_local char g_err[512];

// Record a printf-style message in g_err and return s.
rmsq_status fail(rmsq_status s, const char* fmt, ...);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A buffer's byte range for the overlap check.
struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool output;
  int problem;
  int kind;          // 0 x, 1 residual_in, 2 residual_out, 3 gamma / weights, 4 q / out, 5 scale, 6 bf16
};

// RMSQ_ERR_INVALID_ARG if an output range overlaps any other range (an
// in-place residual, residual_out == residual_in of the same problem, is
// allowed), else RMSQ_OK.
rmsq_status check_overlaps(const Range* rs, int nr);

// True if HIP device dev is a gfx950 GPU (cached per device).
bool device_is_gfx950(int dev);

// Compute units of an MI355X.
constexpr int64_t kComputeUnits = 256;

}  // namespace rmsq_abi
