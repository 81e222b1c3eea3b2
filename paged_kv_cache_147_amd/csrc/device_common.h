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
  return t == PA_F32 ? 4 : (t == PA_F16 || t == PA_BF16) ? 2 : t == PA_FP8_E4M3 ? 1 : 0;
}

// Types the kernels compute with; E4M3 codes are a cache storage type only.
inline bool valid_dtype(pa_dtype t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }
inline bool valid_storage_dtype(pa_dtype t) { return valid_dtype(t) || t == PA_FP8_E4M3; }

// float32 -> 16-bit, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t narrow(F16, float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t narrow(BF16, float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// 16-bit -> float32, exact.
__device__ __forceinline__ float widen1(F16, uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }
__device__ __forceinline__ float widen1(BF16, uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

inline pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace pkv
