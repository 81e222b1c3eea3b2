// Internal: element types, 16-byte chunk helpers and launch checks shared by
// the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

// Storage tags: the kernels move raw bits in 16-byte chunks and widen to
// float32 only where arithmetic happens.
struct F32 { static constexpr int bytes = 4; };
struct F16 { static constexpr int bytes = 2; };
struct BF16 { static constexpr int bytes = 2; };

inline int dtype_bytes(pa_dtype t) {
  return t == PA_F32 ? 4 : (t == PA_F16 || t == PA_BF16) ? 2 : 0;
}

inline bool valid_dtype(pa_dtype t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }

inline pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace pkv
