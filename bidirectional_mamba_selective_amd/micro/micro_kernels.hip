// Microbenchmarks behind the rooflines the benchmark reports (gfx950): the HBM read and copy streams, the
// issue rate of independent fp32 FMAs and of v_exp_f32, the shader clock under that load, and an empty
// kernel for the launch floor.  Built
// into libbimamba_micro.so, a library of its own: the scan library does not contain or call any of it.
// Every entry point enqueues one kernel on `stream` and returns the HIP status; the caller times it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n float4; the sum is written only if it equals a value no input of the benchmark
// produces (the store keeps the loads alive without writing anything in practice).
__global__ __launch_bounds__(256) void k_read(const f32x4* __restrict__ src, size_t n, float* sink) {
  float acc = 0.0f;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const f32x4 v = __builtin_nontemporal_load(src + i);
    acc += (v[0] + v[1]) + (v[2] + v[3]);
  }
  if (acc == -1.2345e37f) sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_copy(const f32x4* __restrict__ src, f32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// 32 independent FMA chains per lane, two steps of each per loop iteration (64 FMAs between loop branches, so
// that the branch costs no issue slots at low occupancy), `iters` iterations: 64 * iters lane-FMAs per thread.
// Every operand is a VGPR (a and b are made lane-varying), the form of the scans' state arithmetic.
// Wavefront 0 of each workgroup records the shader clock (s_memtime) and the 100 MHz reference
// (s_memrealtime) around its loop in clk[2 * block], [2 * block + 1] for the first 4096 workgroups.
__global__ __launch_bounds__(64) void k_fma(float* out, int iters, float a0, float b0, unsigned long long* clk) {
  const float a = a0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  const float b = b0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = static_cast<float>(threadIdx.x + k);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = fmaf(v[k], a, b);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) s += v[k];
  if (s == -1.2345e37f) out[threadIdx.x] = s;
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0 && blockIdx.x < 4096) {
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// The same chains with a wave-uniform multiplier, which the compiler keeps in an SGPR and feeds to
// v_fma_f32 as a scalar operand: mode 0 gives every chain the SGPR operand, mode 1 only the even chains (the
// odd ones keep a lane-varying VGPR multiplier), so SGPR-operand instructions alternate with VGPR-only ones.
__global__ __launch_bounds__(64) void k_fma_sgpr(float* out, int iters, float a0, float b0, int mode) {
  const float av = a0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  const float b = b0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = static_cast<float>(threadIdx.x + k);
  if (mode == 0) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fmaf(v[k], a0, b);
    }
  } else {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fmaf(v[k], (k & 1) ? av : a0, b);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += v[k];
  if (s == -1.2345e37f) out[threadIdx.x] = s;
}

// 8 independent v_exp_f32 chains per lane (each step 2^(v * a), which stays finite for |a| < 1).
__global__ __launch_bounds__(64) void k_exp(float* out, int iters, float a) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.01f * static_cast<float>(threadIdx.x + k);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_amdgcn_exp2f(v[k] * a);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += v[k];
  if (s == -1.2345e37f) out[threadIdx.x] = s;
}

__global__ void k_empty() {}

}  // namespace

extern "C" {

int micro_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_read, dim3(256 * 8 * 4), dim3(256), 0, stream, static_cast<const f32x4*>(src), bytes / 16,
                     sink);
  return static_cast<int>(hipGetLastError());
}

int micro_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  hipLaunchKernelGGL(k_copy, dim3(256 * 8 * 4), dim3(256), 0, stream, static_cast<const f32x4*>(src),
                     static_cast<f32x4*>(dst), bytes / 16);
  return static_cast<int>(hipGetLastError());
}

// waves: wavefronts per SIMD (1024 SIMDs on a 256-CU part), one 64-lane wavefront per workgroup; clk: 8192
// 64-bit counters (see k_fma)
int micro_fma(float* out, int iters, int waves_per_simd, unsigned long long* clk, hipStream_t stream) {
  hipLaunchKernelGGL(k_fma, dim3(1024 * waves_per_simd), dim3(64), 0, stream, out, iters, 0.999f, 0.001f, clk);
  return static_cast<int>(hipGetLastError());
}

// mode 0: every FMA reads an SGPR multiplier; mode 1: every other one (see k_fma_sgpr)
int micro_fma_sgpr(float* out, int iters, int waves_per_simd, int mode, hipStream_t stream) {
  hipLaunchKernelGGL(k_fma_sgpr, dim3(1024 * waves_per_simd), dim3(64), 0, stream, out, iters, 0.999f, 0.001f, mode);
  return static_cast<int>(hipGetLastError());
}

int micro_exp(float* out, int iters, int waves_per_simd, hipStream_t stream) {
  hipLaunchKernelGGL(k_exp, dim3(1024 * waves_per_simd), dim3(64), 0, stream, out, iters, 0.5f);
  return static_cast<int>(hipGetLastError());
}

int micro_empty(int groups, int threads, hipStream_t stream) {
  hipLaunchKernelGGL(k_empty, dim3(groups), dim3(threads), 0, stream);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
