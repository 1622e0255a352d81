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

// log(1 + e^v) = max(v, 0) + log1p(e^-|v|).  log1p(w) on w in (0, 1] uses the
// alternating series w - w^2/2 + w^3/3 - w^4/4 below 2^-5 (truncation below
// w^5/5, i.e. < 3e-7 relative) and log2(1 + w) * ln 2 above it (the rounding
// of 1 + w then costs < 2^-24 / w <= 2e-6 relative).  Both branches are
// evaluated and one is selected, so there is no divergence.
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = fast_exp2(-fabsf(v) * kLog2e);
  const float series = w * (1.0f - w * (0.5f - w * (0.33333334f - w * 0.25f)));
  const float logpath = __builtin_amdgcn_logf(1.0f + w) * kLn2;
  return fmaxf(v, 0.0f) + (w < 0.03125f ? series : logpath);
}

// z * sigmoid(z) = z / (1 + e^-z); e^-z = +inf for very negative z gives -0.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = fast_exp2(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace bimamba
