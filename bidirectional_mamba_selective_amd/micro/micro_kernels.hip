// Microbenchmarks behind the rooflines the benchmark reports (gfx950): the HBM read and copy streams, the
// issue rate of independent fp32 FMAs (with VGPR, SGPR and DPP-broadcast operands) and of v_exp_f32, the
// shader clock under that load, and an empty
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

// The same 32 chains and loop with the multiplier taken in four ways: mode 0 a lane-varying VGPR (as k_fma);
// mode 1 a wave-uniform value, which the compiler keeps in an SGPR and feeds to the FMA as a scalar operand;
// mode 2 that SGPR operand in every other FMA only (the odd chains keep the VGPR); mode 3 a VGPR read through
// the DPP row broadcast (v_fmac_f32_dpp with row_newbcast: every lane of a 16-lane row takes the row's lane k),
// the other way to give every lane one shared value without a copy per lane.  The broadcast source is written
// once before the loop, behind the wait states a DPP read of a VALU result needs.
template <int K>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float m, float b) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(m), "v"(b), "i"(K));
}

template <int MODE>
__global__ __launch_bounds__(64) void k_fma_operand(float* out, int iters, float a0, float b0) {
  const float av = a0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  const float b = b0 * (1.0f + 1e-30f * static_cast<float>(threadIdx.x));
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) v[k] = static_cast<float>(threadIdx.x + k) * 1e-3f;
  if (MODE == 3) asm volatile("s_nop 4" ::: "memory");
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (MODE == 0) {
          v[k] = fmaf(v[k], av, b);
        } else if (MODE == 1) {
          v[k] = fmaf(v[k], a0, b);
        } else if (MODE == 2) {
          v[k] = fmaf(v[k], (k & 1) ? av : a0, b);
        } else {
          switch (k & 3) {  // the multiplier (v += m * b) from lanes 0, 5, 10, 15 of each row
            case 0: fmac_row_bcast<0>(v[k], av, b); break;
            case 1: fmac_row_bcast<5>(v[k], av, b); break;
            case 2: fmac_row_bcast<10>(v[k], av, b); break;
            default: fmac_row_bcast<15>(v[k], av, b); break;
          }
        }
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) s += v[k];
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

// 64 * iters FMAs per thread, one 64-lane wavefront per workgroup, waves_per_simd wavefronts per SIMD; mode:
// 0 VGPR multiplier, 1 SGPR multiplier in every FMA, 2 in every other FMA, 3 DPP row broadcast (see
// k_fma_operand)
int micro_fma_operand(float* out, int iters, int waves_per_simd, int mode, hipStream_t stream) {
  const dim3 grid(1024 * waves_per_simd), block(64);
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_fma_operand<0>, grid, block, 0, stream, out, iters, 0.999f, 0.001f); break;
    case 1: hipLaunchKernelGGL(k_fma_operand<1>, grid, block, 0, stream, out, iters, 0.999f, 0.001f); break;
    case 2: hipLaunchKernelGGL(k_fma_operand<2>, grid, block, 0, stream, out, iters, 0.999f, 0.001f); break;
    case 3: hipLaunchKernelGGL(k_fma_operand<3>, grid, block, 0, stream, out, iters, 0.999f, 0.001f); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
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
