// Device helpers shared by the gfx950 kernels: element formats, cross-lane sums,
// HIP error reporting and per-device properties.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "status.hpp"

namespace pagedkv {

#define PA_HIP_CHECK(expr)                                                          \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess)                                                           \
      return ::pagedkv::fail(PA_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline int elt_bytes(int dtype) { return dtype == PA_F32 ? 4 : dtype == PA_FP8_E4M3 ? 1 : 2; }
inline bool dtype_ok(int dtype) { return dtype == PA_F32 || dtype == PA_F16 || dtype == PA_BF16; }
inline bool pool_dtype_ok(int dtype) { return dtype_ok(dtype) || dtype == PA_FP8_E4M3; }

template <int DT>
constexpr int elt_size() { return DT == PA_F32 ? 4 : DT == PA_FP8_E4M3 ? 1 : 2; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device id).
int device_cus(int* cus);

// Host copy of n elements of device (or pinned host) memory, once the work already ordered
// on `stream` is done (for the debug re-checks only).
template <typename T>
int fetch(std::vector<T>& out, const T* src, size_t n, hipStream_t stream) {
  out.resize(n);
  if (n == 0) return PA_OK;
  PA_HIP_CHECK(hipMemcpyAsync(out.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream));
  PA_HIP_CHECK(hipStreamSynchronize(stream));
  return PA_OK;
}

// Debug re-checks (see debug_checks()): the slots inside [0, num_slots) are distinct; the
// copy pairs inside [0, num_blocks) have distinct destinations and no block is both a
// source and a destination. PA_EINVAL names the first offender.
int check_slots(const int64_t* slots, int32_t n, int64_t num_slots, hipStream_t stream);
int check_pairs(const int32_t* pairs, int32_t n, int32_t num_blocks, hipStream_t stream);

// ---- element formats -------------------------------------------------------

// 16 bytes of storage = 4 fp32, 8 fp16 / bf16 or 16 E4M3 values, widened exactly to fp32.
// E4M3 uses gfx950's conversion instruction, which reads the OCP E4M3 format.
template <int DT>
__device__ __forceinline__ void widen16(const uint4& x, float* f) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (DT == PA_FP8_E4M3) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      f[4 * i] = lo.x;
      f[4 * i + 1] = lo.y;
      f[4 * i + 2] = hi.x;
      f[4 * i + 3] = hi.y;
    }
  } else if constexpr (DT == PA_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == PA_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> OCP E4M3 code: round to nearest, ties to even, magnitudes >= 448 saturate to
// 448, NaN -> 0x7F, the sign of values rounding to zero kept. Bit operations only, so
// the code is the same on every device (E4M3: bias 7, 3 mantissa bits, smallest normal
// 2^-6, subnormal steps of 2^-9).
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;            // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;     // >= 448, infinities included
  if (a >= 0x3c800000u) {                         // >= 2^-6: normal
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // keep 3 mantissa bits, RNE
    const uint32_t code = (r >> 20) - (120u << 3);        // exponent bias 127 -> 7
    return sign | (code > 0x7eu ? 0x7eu : code);
  }
  // below 2^-6: multiples of 2^-9 (the scaling by 512 is exact), nearest even
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

// 4 fp32 (or 8 for 16-bit formats) -> 16 bytes of storage, round to nearest even.
template <int DT>
__device__ __forceinline__ uint4 narrow16(const float* f) {
  uint32_t w[4];
  if constexpr (DT == PA_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
  } else if constexpr (DT == PA_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i]);
      uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i + 1]);
      w[i] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_bits_rne(f[2 * i]) | (bf16_bits_rne(f[2 * i + 1]) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---- cross-lane sums -------------------------------------------------------

// DPP move within a row of 16 lanes; every source lane is active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPR lanes (LPR = 4, 8, 16 or 32); every lane of a
// group receives the group's sum. The order of additions is fixed.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "group width");
  x += dpp_f<0xB1>(x);                              // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);                              // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_f<0x141>(x);     // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_f<0x140>(x);    // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

}  // namespace pagedkv
