// Chunked bidirectional selective scan for gfx950.
//
// Operation: "DiffuMamba: High-Throughput Diffusion LMs with Mamba Backbone"
// (arXiv v4), Section 3.2 eq. (4)-(6), with the selective discretisation
// delta = softplus(dt + dt_bias), abar = exp(delta * A), input delta * x * B,
// readout C . h + D * x per direction, and the SiLU(z) gate on the sum.
//
// Work decomposition (one lane = one channel d, all d_state states in
// registers; one wavefront = 64 channels of one chunk of one sequence):
//   k_summary  walks each chunk backwards and produces, per (chunk, d, n):
//              Sf = forward state at the chunk end starting from zero,
//              Sr = reverse state at the chunk start starting from zero,
//              P  = product of abar over the chunk,
//              and the zero-started reverse state at every sub-chunk boundary
//              together with the suffix sum of delta to the chunk end.
//   k_carry    composes the affine chunk maps h -> P h + S in both directions:
//              Cf[c] = forward state entering chunk c, Cr[c] = reverse state
//              entering chunk c from the right.
//   k_output   walks each chunk forwards one sub-chunk of 16 tokens at a time.
//              For every state n it forms abar and delta*x*B once per token,
//              runs the forward recurrence from the carried state and the
//              reverse recurrence from the exact boundary state, and
//              accumulates C . (h_fwd + h_rev) per token; then adds the skip
//              term, applies the gate and stores.
// The transition is diagonal per (d, n), so nothing here is a dense
// contraction; the kernels are bound by VALU/transcendental issue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "launch.h"

namespace bimamba {

template <typename T>
__device__ __forceinline__ float ld(const T* __restrict__ p, size_t i) {
  return to_f32(p[i]);
}

// ---------------------------------------------------------------------------
// Tile loading: SUB consecutive tokens of one channel per lane (coalesced across
// the 64 lanes of a wavefront), all loads issued together.
// ---------------------------------------------------------------------------
template <typename T, int SUB>
__device__ __forceinline__ void load_tile(const T* __restrict__ p, size_t base, int D, int nvalid, float (&v)[SUB]) {
  // Addresses are clamped into the valid range and the surplus values zeroed
  // afterwards, so the loads carry no branches and are all in flight at once.
#pragma unroll
  for (int k = 0; k < SUB; ++k) v[k] = ld(p, base + static_cast<size_t>(min(k, nvalid - 1)) * D);
#pragma unroll
  for (int k = 0; k < SUB; ++k) v[k] = k < nvalid ? v[k] : 0.0f;
}

// Stage a [SUB x N] tile of a token-major [*, N] matrix into LDS as fp32 [NM][SUB]
// (state-major, so a state's SUB values are contiguous); missing tokens and
// states >= N become 0.
template <typename T, int NM, int SUB>
__device__ __forceinline__ void stage_bc(const T* __restrict__ M, size_t row0, int N, int nvalid, float (*dst)[SUB],
                                         int lane) {
  constexpr int PER = (NM * SUB + 63) / 64;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * 64 + lane;
    const int k = e / NM;
    const int n = e - k * NM;
    v[i] = ld(M, (row0 + min(k, nvalid - 1)) * N + min(n, N - 1));
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * 64 + lane;
    const int k = e / NM;
    const int n = e - k * NM;
    if (e < NM * SUB) dst[n][k] = (k < nvalid && n < N) ? v[i] : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// k_summary: grid (d_inner / 64, nchunk, batch), block 64.
// Walks the chunk's tiles from right to left.  Per state n and tile it forms
// abar and delta*x*B once per token, runs the tile-local forward recurrence
// from zero (composed into the chunk's forward end state with the decay of
// everything to the right of the tile) and continues the reverse recurrence
// from the running state; the running reverse state is stored at every tile
// boundary.
// ---------------------------------------------------------------------------
template <typename T, int NM>
__global__ __launch_bounds__(64) void k_summary(const T* __restrict__ x, const T* __restrict__ dt,
                                                const float* __restrict__ A, const T* __restrict__ Bm,
                                                const float* __restrict__ dt_bias, int L, int D, int N, int chunk,
                                                int nchunk, int nsub, float* __restrict__ Sf,
                                                float* __restrict__ Sr, float* __restrict__ P,
                                                float* __restrict__ R, float* __restrict__ SIG) {
  constexpr int SUB = static_cast<int>(kSub);
  __shared__ float sB[NM][SUB];
  __shared__ float sA2[NM][64];
  __shared__ float sR[NM][64];
  __shared__ float sS[NM][64];
  const int lane = threadIdx.x;
  const int d = blockIdx.x * 64 + lane;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int t0 = c * chunk;
  const int te = min(L, t0 + chunk);
  const size_t row = static_cast<size_t>(b) * L;
  const size_t cbase = static_cast<size_t>(b) * nchunk + c;

  for (int n = 0; n < N; ++n) {
    sA2[n][lane] = A[static_cast<size_t>(d) * N + n] * kLog2e;
    sR[n][lane] = 0.0f;
    sS[n][lane] = 0.0f;
  }
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  float sigma = 0.0f;  // sum of delta from the current tile's right edge to the chunk end

  const int nsub_c = (te - t0 + SUB - 1) / SUB;
  for (int j = nsub_c - 1; j >= 0; --j) {
    const int ts = t0 + j * SUB;
    const int nvalid = min(SUB, te - ts);
    float xr[SUB], dr[SUB];
    load_tile<T, SUB>(x, (row + ts) * D + d, D, nvalid, xr);
    load_tile<T, SUB>(dt, (row + ts) * D + d, D, nvalid, dr);
    __syncthreads();  // previous tile's reads of sB are done
    stage_bc<T, NM, SUB>(Bm, row + ts, N, nvalid, sB, lane);
    float dl[SUB], u[SUB];
    float tile_sum = 0.0f;
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      dl[k] = k < nvalid ? softplus_f32(dr[k] + bias) : 0.0f;
      u[k] = dl[k] * xr[k];
      tile_sum += dl[k];
    }
    __syncthreads();
    const size_t jb = cbase * nsub + (j - 1);
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
      const float a2 = sA2[n][lane];
      float r = sR[n][lane];
      float a[SUB], bb[SUB];
      float f = 0.0f;
#pragma unroll
      for (int k = 0; k < SUB; ++k) {
        a[k] = fast_exp2(dl[k] * a2);
        bb[k] = u[k] * sB[n][k];
        f = fmaf(a[k], f, bb[k]);
      }
#pragma unroll
      for (int k = SUB - 1; k >= 0; --k) r = fmaf(a[k], r, bb[k]);
      sS[n][lane] = fmaf(fast_exp2(a2 * sigma), f, sS[n][lane]);
      sR[n][lane] = r;
      if (j > 0) R[(jb * N + n) * D + d] = r;
    }
    sigma += tile_sum;
    if (j > 0) SIG[jb * D + d] = sigma;
  }
  for (int n = 0; n < N; ++n) {
    const size_t o = (cbase * N + n) * D + d;
    Sf[o] = sS[n][lane];
    Sr[o] = sR[n][lane];
    P[o] = fast_exp2(sA2[n][lane] * sigma);
  }
}

// ---------------------------------------------------------------------------
// k_carry: one thread per (b, n, d); sequential over chunks in both directions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_carry(const float* __restrict__ Sf, const float* __restrict__ Sr,
                                               const float* __restrict__ P, float* __restrict__ Cf,
                                               float* __restrict__ Cr, const float* __restrict__ h_in, int batch,
                                               int nchunk, int N, int D) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t total = static_cast<size_t>(batch) * N * D;
  if (idx >= total) return;
  const int d = static_cast<int>(idx % D);
  const int n = static_cast<int>((idx / D) % N);
  const int b = static_cast<int>(idx / (static_cast<size_t>(D) * N));
  float cf = h_in ? h_in[(static_cast<size_t>(b) * D + d) * N + n] : 0.0f;
  for (int c = 0; c < nchunk; ++c) {
    const size_t o = ((static_cast<size_t>(b) * nchunk + c) * N + n) * D + d;
    Cf[o] = cf;
    cf = fmaf(P[o], cf, Sf[o]);
  }
  float cr = 0.0f;
  for (int c = nchunk - 1; c >= 0; --c) {
    const size_t o = ((static_cast<size_t>(b) * nchunk + c) * N + n) * D + d;
    Cr[o] = cr;
    cr = fmaf(P[o], cr, Sr[o]);
  }
}

// ---------------------------------------------------------------------------
// k_output: grid (d_inner / 64, nchunk, batch), block 64.
// DIRS: bit 0 = forward readout, bit 1 = reverse readout.
// ---------------------------------------------------------------------------
template <typename T, int NM, int DIRS>
__global__ __launch_bounds__(64) void k_output(const T* __restrict__ x, const T* __restrict__ dt,
                                               const T* __restrict__ z, const float* __restrict__ A,
                                               const T* __restrict__ Bm, const T* __restrict__ Cm,
                                               const float* __restrict__ Dv, const float* __restrict__ dt_bias,
                                               T* __restrict__ out, int L, int D, int N, int chunk, int nchunk,
                                               int nsub, int gate, const float* __restrict__ Cf,
                                               const float* __restrict__ Cr, const float* __restrict__ R,
                                               const float* __restrict__ SIG, float* __restrict__ h_out) {
  constexpr int SUB = static_cast<int>(kSub);
  __shared__ float sB[NM][SUB];
  __shared__ float sC[NM][SUB];
  // per-lane state, indexed by a runtime state index
  __shared__ float sA2[NM][64];
  __shared__ float sHf[NM][64];
  __shared__ float sHr[NM][64];
  __shared__ float sCr[NM][64];
  const int lane = threadIdx.x;
  const int d = blockIdx.x * 64 + lane;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int t0 = c * chunk;
  const int te = min(L, t0 + chunk);
  const size_t row = static_cast<size_t>(b) * L;
  const size_t cbase = static_cast<size_t>(b) * nchunk + c;

  for (int n = 0; n < N; ++n) {
    sA2[n][lane] = A[static_cast<size_t>(d) * N + n] * kLog2e;
    sHf[n][lane] = Cf[(cbase * N + n) * D + d];
    sCr[n][lane] = Cr[(cbase * N + n) * D + d];
  }
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  constexpr float ndir = (DIRS == 3) ? 2.0f : 1.0f;
  const float skip = Dv ? ndir * Dv[d] : 0.0f;

  const int nsub_c = (te - t0 + SUB - 1) / SUB;
  for (int j = 0; j < nsub_c; ++j) {
    const int ts = t0 + j * SUB;
    const int nvalid = min(SUB, te - ts);
    const bool last = (j == nsub_c - 1);
    const size_t jb = cbase * nsub + j;
    // every load of the tile is issued before any of it is used
    float xr[SUB], dr[SUB], zr[SUB], rj[NM];
    load_tile<T, SUB>(x, (row + ts) * D + d, D, nvalid, xr);
    load_tile<T, SUB>(dt, (row + ts) * D + d, D, nvalid, dr);
    if (gate) load_tile<T, SUB>(z, (row + ts) * D + d, D, nvalid, zr);
    // the slot of the last tile is inside the allocation but never written: load and discard
#pragma unroll
    for (int n = 0; n < NM; ++n) rj[n] = R[(jb * N + min(n, N - 1)) * D + d];
#pragma unroll
    for (int n = 0; n < NM; ++n) rj[n] = (!last && n < N) ? rj[n] : 0.0f;
    const float sj0 = SIG[jb * D + d];
    const float sj = last ? 0.0f : sj0;
    __syncthreads();  // previous tile's reads of sB / sC / sHr are done
    stage_bc<T, NM, SUB>(Bm, row + ts, N, nvalid, sB, lane);
    stage_bc<T, NM, SUB>(Cm, row + ts, N, nvalid, sC, lane);
    float dl[SUB], u[SUB], y[SUB];
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      dl[k] = k < nvalid ? softplus_f32(dr[k] + bias) : 0.0f;
      u[k] = dl[k] * xr[k];
      y[k] = skip * xr[k];
    }
    if (DIRS & 2) {
      // exact reverse state entering this tile from the right
#pragma unroll
      for (int n = 0; n < NM; ++n)
        if (n < N) sHr[n][lane] = fmaf(fast_exp2(sA2[n][lane] * sj), sCr[n][lane], rj[n]);
    }
    __syncthreads();
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
      const float a2 = sA2[n][lane];
      float hf = sHf[n][lane];
      float a[SUB], bb[SUB];
#pragma unroll
      for (int k = 0; k < SUB; ++k) {
        a[k] = fast_exp2(dl[k] * a2);
        bb[k] = u[k] * sB[n][k];
        hf = fmaf(a[k], hf, bb[k]);
        if (DIRS & 1) y[k] = fmaf(sC[n][k], hf, y[k]);
      }
      sHf[n][lane] = hf;
      if (DIRS & 2) {
        float hr = sHr[n][lane];
#pragma unroll
        for (int k = SUB - 1; k >= 0; --k) {
          hr = fmaf(a[k], hr, bb[k]);
          y[k] = fmaf(sC[n][k], hr, y[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      if (k < nvalid) {
        const float o = gate ? y[k] * silu_f32(zr[k]) : y[k];
        from_f32(o, out + (row + ts + k) * D + d);
      }
    }
  }
  if (h_out != nullptr && c == nchunk - 1) {
    for (int n = 0; n < N; ++n) h_out[(static_cast<size_t>(b) * D + d) * N + n] = sHf[n][lane];
  }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <typename T, int NM>
static hipError_t launch_typed(const ScanArgs& a, const Plan& p, void* ws, hipStream_t stream, int stage) {
  char* w = static_cast<char*>(ws);
  float* Sf = reinterpret_cast<float*>(w + p.off_sf);
  float* Sr = reinterpret_cast<float*>(w + p.off_sr);
  float* P = reinterpret_cast<float*>(w + p.off_p);
  float* Cf = reinterpret_cast<float*>(w + p.off_cf);
  float* Cr = reinterpret_cast<float*>(w + p.off_cr);
  float* R = reinterpret_cast<float*>(w + p.off_r);
  float* SIG = reinterpret_cast<float*>(w + p.off_sig);
  const int L = static_cast<int>(p.seqlen), D = static_cast<int>(p.d_inner), N = static_cast<int>(p.d_state);
  const int chunk = static_cast<int>(p.chunk), nchunk = static_cast<int>(p.nchunk), nsub = static_cast<int>(p.nsub);
  const dim3 grid(static_cast<unsigned>(D / 64), static_cast<unsigned>(nchunk), static_cast<unsigned>(p.batch));
  const T* x = static_cast<const T*>(a.x);
  const T* dt = static_cast<const T*>(a.dt);
  const T* z = static_cast<const T*>(a.z);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  T* out = static_cast<T*>(a.out);

  hipError_t e = hipSuccess;
  if (stage < 0 || stage == 0) {
    hipLaunchKernelGGL((k_summary<T, NM>), grid, dim3(64), 0, stream, x, dt, a.A, Bm, a.dt_bias, L, D, N, chunk,
                       nchunk, nsub, Sf, Sr, P, R, SIG);
    e = hipGetLastError();
    if (e != hipSuccess || stage == 0) return e;
  }

  if (stage < 0 || stage == 1) {
    const size_t nthreads = static_cast<size_t>(p.batch) * N * D;
    hipLaunchKernelGGL(k_carry, dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0, stream, Sf, Sr,
                       P, Cf, Cr, a.h_in, static_cast<int>(p.batch), nchunk, N, D);
    e = hipGetLastError();
    if (e != hipSuccess || stage == 1) return e;
  }

  const int gate = (a.flags & kNoGate) ? 0 : 1;
  if (a.flags & kFwdOnly) {
    hipLaunchKernelGGL((k_output<T, NM, 1>), grid, dim3(64), 0, stream, x, dt, z, a.A, Bm, Cm, a.D, a.dt_bias, out,
                       L, D, N, chunk, nchunk, nsub, gate, Cf, Cr, R, SIG, a.h_out);
  } else if (a.flags & kRevOnly) {
    hipLaunchKernelGGL((k_output<T, NM, 2>), grid, dim3(64), 0, stream, x, dt, z, a.A, Bm, Cm, a.D, a.dt_bias, out,
                       L, D, N, chunk, nchunk, nsub, gate, Cf, Cr, R, SIG, a.h_out);
  } else {
    hipLaunchKernelGGL((k_output<T, NM, 3>), grid, dim3(64), 0, stream, x, dt, z, a.A, Bm, Cm, a.D, a.dt_bias, out,
                       L, D, N, chunk, nchunk, nsub, gate, Cf, Cr, R, SIG, a.h_out);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dtype(const ScanArgs& a, const Plan& p, void* ws, hipStream_t stream, int stage) {
  if (p.d_state <= 4) return launch_typed<T, 4>(a, p, ws, stream, stage);
  if (p.d_state <= 8) return launch_typed<T, 8>(a, p, ws, stream, stage);
  return launch_typed<T, 16>(a, p, ws, stream, stage);
}

hipError_t launch_chunked(const ScanArgs& a, const Plan& p, void* workspace, hipStream_t stream, int stage) {
  if (a.io_dtype == 1) return launch_dtype<bf16_t>(a, p, workspace, stream, stage);
  return launch_dtype<float>(a, p, workspace, stream, stage);
}

}  // namespace bimamba
