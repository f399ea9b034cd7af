// Internal helpers shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specsam.h"

namespace specsam {

// Records the message returned by ss_last_error_string() and passes rc on.
int set_error(int rc, const char* fmt, ...);

// Checks a launch: SS_OK, or SS_ELAUNCH with the HIP error text recorded.
int check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Wave-wide reductions over 64 lanes (butterfly through cross-lane shuffles;
// every lane ends with the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the wave (Hillis-Steele through shuffles).
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    float t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace specsam
