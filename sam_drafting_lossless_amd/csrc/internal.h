// Internal helpers shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

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

// Cross-lane moves through DPP (the GFX9 encodings gfx950 keeps), for code
// in which all 64 lanes of the wavefront are active. A lane whose source
// lies outside its 16-lane row (or the wavefront), or whose row is masked
// off, receives `id`. Unlike shuffles through ds_bpermute these stay in the
// vector ALU.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int id, int v) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float id, float v) {
  return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(id), __float_as_int(v)));
}

// A double moves as its two 32-bit halves under the same control.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_d(double id, double v) {
  const unsigned long long vi = (unsigned long long)__double_as_longlong(v);
  const unsigned long long ii = (unsigned long long)__double_as_longlong(id);
  const unsigned lo = (unsigned)dpp_i<CTRL, ROW_MASK>((int)(unsigned)ii, (int)(unsigned)vi);
  const unsigned hi =
      (unsigned)dpp_i<CTRL, ROW_MASK>((int)(unsigned)(ii >> 32), (int)(unsigned)(vi >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const unsigned long long x = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

// Inclusive scan of an associative, commutative operation with identity id:
// shifts by 1, 2, 4 and 8 inside each row, then the row broadcasts of lanes
// 15 and 31.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan(T v, T id, Op op) {
  if constexpr (std::is_same<T, double>::value) {
    v = op(v, dpp_d<kDppRowShr1>(id, v));
    v = op(v, dpp_d<kDppRowShr2>(id, v));
    v = op(v, dpp_d<kDppRowShr4>(id, v));
    v = op(v, dpp_d<kDppRowShr8>(id, v));
    v = op(v, dpp_d<kDppRowBcast15, 0xa>(id, v));
    v = op(v, dpp_d<kDppRowBcast31, 0xc>(id, v));
  } else if constexpr (std::is_same<T, int>::value) {
    v = op(v, dpp_i<kDppRowShr1>(id, v));
    v = op(v, dpp_i<kDppRowShr2>(id, v));
    v = op(v, dpp_i<kDppRowShr4>(id, v));
    v = op(v, dpp_i<kDppRowShr8>(id, v));
    v = op(v, dpp_i<kDppRowBcast15, 0xa>(id, v));
    v = op(v, dpp_i<kDppRowBcast31, 0xc>(id, v));
  } else {
    v = op(v, dpp_f<kDppRowShr1>(id, v));
    v = op(v, dpp_f<kDppRowShr2>(id, v));
    v = op(v, dpp_f<kDppRowShr4>(id, v));
    v = op(v, dpp_f<kDppRowShr8>(id, v));
    v = op(v, dpp_f<kDppRowBcast15, 0xa>(id, v));
    v = op(v, dpp_f<kDppRowBcast31, 0xc>(id, v));
  }
  return v;
}

// Inclusive prefix sum across the wavefront.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  return wave_scan(v, 0.0f, [](float x, float y) { return x + y; });
}

// N independent wavefront inclusive sums, each step taken on all N values
// before the next, so that their shuffles overlap (one after another, each
// sum's chain of dependent steps is exposed when a SIMD runs one
// wavefront). Each value gets exactly wave_inclusive_sum's additions.
template <int N>
__device__ __forceinline__ void wave_inclusive_sum_n(float (&v)[N]) {
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowShr1>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowShr2>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowShr4>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowShr8>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowBcast15, 0xa>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = dpp_f<kDppRowBcast31, 0xc>(0.0f, v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += t[i];
}

// The value of the previous lane (0 in lane 0): an inclusive scan's
// exclusive counterpart, bit for bit.
__device__ __forceinline__ float wave_shift_up1(float v) {
  return dpp_f<kDppWaveShr1>(0.0f, v);
}

// The same in double precision (the draw's running sums).
__device__ __forceinline__ double wave_inclusive_sum_d(double v) {
  return wave_scan(v, 0.0, [](double x, double y) { return x + y; });
}
__device__ __forceinline__ double wave_shift_up1_d(double v) {
  return dpp_d<kDppWaveShr1>(0.0, v);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  return readlane_d(wave_inclusive_sum_d(v), 63);
}

// An empty asm that reads and writes v, so that v is computed where it
// stands: a sum used only after a loop with conditional stores is otherwise
// sunk below the loop, and every input of it is held until then.
__device__ __forceinline__ void keep_here(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void keep_here(u32x4& v) { asm volatile("" : "+v"(v)); }
// The same for a wavefront-uniform value, kept in a scalar register.
__device__ __forceinline__ void keep_here_uniform(int& v) { asm volatile("" : "+s"(v)); }

// Mask of the lanes where b holds. The compiler's own ballot takes an int
// and materialises the compare first; this one uses the compare's mask.
__device__ __forceinline__ unsigned long long ballot_mask(bool b) {
  return __builtin_amdgcn_ballot_w64(b);
}

// Number of lanes below this one whose bit is set in a wavefront mask.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Wavefront reductions; every lane ends with the result.
__device__ __forceinline__ float wave_sum(float v) { return lane63(wave_inclusive_sum(v)); }

__device__ __forceinline__ float wave_max(float v) {
  return lane63(wave_scan(v, -INFINITY, [](float x, float y) { return fmaxf(x, y); }));
}

__device__ __forceinline__ int wave_or(int v) {
  return lane63(wave_scan(v, 0, [](int x, int y) { return x | y; }));
}

__device__ __forceinline__ int wave_max_i(int v) {
  return lane63(wave_scan(v, INT_MIN, [](int x, int y) { return x > y ? x : y; }));
}

__device__ __forceinline__ int wave_min_i(int v) {
  return lane63(wave_scan(v, INT_MAX, [](int x, int y) { return x < y ? x : y; }));
}

// Reduces (x, y) pairs with merge(x, y, ox, oy), an associative and
// commutative update of (x, y) by (ox, oy) with identity (idx, idy); y is
// carried as raw 32-bit bits. Every lane ends with the result.
template <typename Merge>
__device__ __forceinline__ void wave_reduce2(float& x, float& y, float idx, float idy,
                                             Merge merge) {
#define SPECSAM_DPP2(C, M)                                        \
  {                                                               \
    const float ox = dpp_f<C, M>(idx, x), oy = dpp_f<C, M>(idy, y); \
    merge(x, y, ox, oy);                                          \
  }
  SPECSAM_DPP2(kDppRowShr1, 0xf)
  SPECSAM_DPP2(kDppRowShr2, 0xf)
  SPECSAM_DPP2(kDppRowShr4, 0xf)
  SPECSAM_DPP2(kDppRowShr8, 0xf)
  SPECSAM_DPP2(kDppRowBcast15, 0xa)
  SPECSAM_DPP2(kDppRowBcast31, 0xc)
#undef SPECSAM_DPP2
  x = lane63(x);
  y = lane63(y);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace specsam
