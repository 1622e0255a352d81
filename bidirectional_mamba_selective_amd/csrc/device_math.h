// Device-side helpers shared by the scan kernels: I/O element conversion and the
// per-(token, channel) activations.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bimamba {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v.bits) << 16); }

__device__ __forceinline__ void from_f32(float v, float* dst) { *dst = v; }
// Round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ void from_f32(float v, bf16_t* dst) {
  dst->bits = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// log(1 + e^v) = max(v, 0) + log1p(w) with w = e^-|v| in (0, 1].  s = 1 + w is
// rounded; its rounding error c = (s - 1) - w is exact (s - 1 is exact for s in
// [1, 2], and so is the error of the sum), so log1p(w) = ln(s - c) =
// ln(s) - c/s + O(c^2).  c/s is taken as c (2 - s) = c - c (s - 1), off by
// c (s - 1)^2 / s, below 2^-24 of log1p(w).  v_log_f32 is within 1 ulp on [1, 2)
// (checked on every float there), which leaves log1p(w) within ~1.3e-7 relative.
// No branch and no select.
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = fast_exp2(-fabsf(v) * kLog2e);
  const float s = 1.0f + w;
  const float sm1 = s - 1.0f;
  const float c = sm1 - w;
  return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(s), kLn2, fmaf(c, sm1, -c));
}

// z * sigmoid(z) = z / (1 + e^-z); e^-z = +inf for very negative z gives -0.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = fast_exp2(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace bimamba
