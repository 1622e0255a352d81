// Chunked bidirectional selective scan for gfx950.
//
// Operation: "DiffuMamba: High-Throughput Diffusion LMs with Mamba Backbone"
// (arXiv v4), Section 3.2 eq. (4)-(6), with the selective discretisation
// delta = softplus(dt + dt_bias), abar = exp(delta * A), input delta * x * B,
// readout C . h + D * x per direction, and the SiLU(z) gate on the sum.
//
// Work decomposition (one lane = one channel d; one wavefront = 64 channels
// of one chunk of one sequence; a chunk is walked in tiles of kSub tokens that
// sit in registers):
//   k_stage_bc copies B and C into an fp32 table laid out per tile and state
//              (kSub values of B, then kSub of C; zero past the sequence end).
//              B and C do not depend on the channel: the output pass and the
//              general-A summary read them with wave-uniform scalar loads into
//              SGPRs, which VALU instructions take as operands, so they hold
//              no vector registers (the saving buys a wavefront per SIMD).  The
//              geometric-A summary, whose state step is too short to hide a
//              scalar load's wait, copies each tile's B rows into LDS instead.
//   k_summary  walks each chunk's tiles right to left.  Per state n and tile it
//              forms abar and delta*x*B once per token, runs the tile-local
//              forward recurrence from zero (composed into the chunk's forward
//              end state with the decay of everything to the tile's right) and
//              continues the reverse recurrence from the running state, which
//              (when both directions are kept) it stores at every tile
//              boundary together with the suffix sum of delta to the chunk
//              end.  Outputs per (chunk, d, n):
//              Sf = forward end state from zero, Sr = reverse start state from
//              zero, P = product of abar over the chunk.
//   k_carry    composes the affine chunk maps h -> P h + S in both directions:
//              Cf[c] = forward state entering chunk c, Cr[c] = reverse state
//              entering chunk c from the right.
//   k_output   walks each chunk's tiles left to right.  Per state n it forms
//              abar and delta*x*B once per token and shares them between the
//              forward recurrence (from the carried state) and the reverse
//              recurrence (from the exact boundary state), accumulating
//              C . (h_fwd + h_rev) per token; then skip term, gate, store.  A
//              reverse-only pass walks the tiles right to left instead and
//              carries its reverse state from tile to tile.
//   k_block    a whole short block of block-cache decoding in one kernel
//              (blocks of up to 16 tokens, and of 65 to 128, in two halves).
//   k_block_parts  the same for blocks of 17 to 64 tokens, cut into parts of
//              16 tokens whose chains run from zero side by side and are
//              corrected afterwards by the decayed entering states.
// The transition is diagonal per (d, n), so nothing here is a dense
// contraction; the kernels are bound by VALU and transcendental issue.
//
// Per-channel geometric A.  When a channel's row satisfies A[d,n] = (n+1) A[d,0]
// exactly (the S4D-real initialisation has this form), exp(delta A[d,n]) is
// the (n+1)-th power of r = exp(delta A[d,0]); the kernels then form abar by
// one multiplication per state instead of one exponential.  The test is exact
// and per wavefront; any other A takes the general path.  Both bodies sit in
// one kernel behind a wavefront-uniform branch, so one launch serves any mix.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "launch.h"

namespace bimamba {

// ---------------------------------------------------------------------------
// Buffer-resource I/O.  A tile's base address goes into the resource, the
// lane's channel into the VGPR offset and the token row into the SGPR offset,
// so loads and stores need no per-lane address arithmetic.
// ---------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor, untyped 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7fffffffull ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, kRsrcWord3);
}

// Cache policy for data read or written exactly once (activations, outputs,
// boundary states): non-temporal, the nt bit of the buffer instruction's
// cache-policy field, so that these streams do not push data that is read
// again (chunk carries, the B/C table) out of L2.
constexpr int kStreamCpol = 2;

template <typename T>
struct IO;

template <>
struct IO<float> {
  static constexpr uint32_t kBytes = 4;
  template <int CP = 0>
  static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP));
  }
  template <int CP = 0>
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, CP);
  }
};


template <>
struct IO<bf16_t> {
  static constexpr uint32_t kBytes = 2;
  template <int CP = 0>
  static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, CP);
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
  // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN
  template <int CP = 0>
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const __bf16 h = static_cast<__bf16>(v);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), r, voff, soff, CP);
  }
};

// v[k] = tile row k of this lane's channel; rows past nvalid repeat the last
// valid row (their values are never used).  Row offsets are clamped so that
// every load is in bounds and none is guarded by a branch: all of them are in
// flight together.
template <typename T, int SUB>
__device__ __forceinline__ void load_col_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t row_bytes, int nvalid,
                                             float (&v)[SUB]) {
#pragma unroll
  for (int k = 0; k < SUB; ++k)
    v[k] = IO<T>::template load<kStreamCpol>(r, voff, static_cast<uint32_t>(min(k, nvalid - 1)) * row_bytes);
}

// delta = softplus(dt + dt_bias) for a tile's tokens; tokens past nvalid get
// delta = 0 (abar = 1 and no input: they leave the states unchanged).  Full
// tiles take a path without the per-token test, which the compiler would turn
// into a branch around each softplus.
template <int SUB>
__device__ __forceinline__ void tile_delta(const float (&dr)[SUB], float bias, int nvalid, float (&dl)[SUB]) {
  if (nvalid == SUB) {
#pragma unroll
    for (int k = 0; k < SUB; ++k) dl[k] = softplus_f32(dr[k] + bias);
  } else {
#pragma unroll
    for (int k = 0; k < SUB; ++k) dl[k] = k < nvalid ? softplus_f32(dr[k] + bias) : 0.0f;
  }
}

// Store rows k < nvalid of a tile column (full tiles without per-row tests).
template <typename T, int SUB>
__device__ __forceinline__ void store_col(const float (&v)[SUB], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t row_bytes, int nvalid) {
  if (nvalid == SUB) {
#pragma unroll
    for (int k = 0; k < SUB; ++k) IO<T>::template store<kStreamCpol>(v[k], r, voff, static_cast<uint32_t>(k) * row_bytes);
  } else {
#pragma unroll
    for (int k = 0; k < SUB; ++k)
      if (k < nvalid) IO<T>::template store<kStreamCpol>(v[k], r, voff, static_cast<uint32_t>(k) * row_bytes);
  }
}

// Loads through a constant-address-space pointer with a wave-uniform address
// become scalar loads into SGPRs.  Only for memory no kernel in flight writes.
typedef const float __attribute__((address_space(4))) sfloat;

__device__ __forceinline__ const sfloat* scalar_ptr(const float* p) { return (const sfloat*)p; }

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_f32<bf16_t>(const bf16_t* p) { return to_f32(*p); }

// ---------------------------------------------------------------------------
// k_stage_bc: one thread per (batch, tile, state, token of the tile).
// bct[((b * ntile + g) * N + n) * 2 * kSub + {k, kSub + k}] = {B, C}[b, g * kSub + k, n].
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_stage_bc(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                  float* __restrict__ bct, int L, int N, int ntile, size_t total) {
  constexpr int SUB = static_cast<int>(kSub);
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int k = static_cast<int>(idx % SUB);
  const size_t rest = idx / SUB;
  const int n = static_cast<int>(rest % N);
  const size_t bg = rest / N;  // b * ntile + g
  const int g = static_cast<int>(bg % ntile);
  const size_t b = bg / ntile;
  const int t = g * SUB + k;
  float bv = 0.0f, cv = 0.0f;
  if (t < L) {
    const size_t src = (b * L + t) * N + n;
    bv = ld_f32(Bm + src);
    cv = ld_f32(Cm + src);
  }
  float* dst = bct + rest * 2 * SUB;
  dst[k] = bv;
  dst[SUB + k] = cv;
}

// Whether every lane's A row is geometric: A[d,n] == (n+1) * A[d,0] exactly.
__device__ __forceinline__ bool wave_geometric(bool lane_geo) { return __all(lane_geo ? 1 : 0) != 0; }

// ---------------------------------------------------------------------------
// Explicit waits.  The tile buffers are filled by direct-to-LDS buffer loads,
// whose completion the compiler does not track: the kernel waits for them
// itself.  The memory clobber keeps the compiler from moving LDS accesses
// across a wait.
// ---------------------------------------------------------------------------
// s_waitcnt vmcnt(0) through the builtin, so that the compiler's own wait insertion knows that every
// vector memory operation issued so far is complete (with an opaque asm wait it kept adding waits of
// its own for loads already waited for: 1-2 % of the output pass); the empty asm keeps memory accesses
// from moving across it.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt at their maxima (not waited for)
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Direct-to-LDS load of a [kSub x 64] tile of a token-major [*, D] tensor
// (base = the tile's first row at this wavefront's first channel) into dst,
// laid out [row][lane].  One instruction moves 16 bytes per lane, i.e. 1 KiB:
// 8 rows of bf16 or 4 rows of fp32.  Rows past nvalid repeat the last valid
// row (they are never used), so every read is in bounds.
template <typename T>
__device__ __forceinline__ void lds_load_tile(const T* base, int nvalid, uint32_t row_bytes, T (*dst)[64],
                                              int lane) {
  constexpr int kLanesPerRow = 64 * static_cast<int>(sizeof(T)) / 16;
  constexpr int kRowsPerInst = 64 / kLanesPerRow;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, static_cast<size_t>(nvalid) * row_bytes);
  const int rl = lane / kLanesPerRow;
  const uint32_t cb = static_cast<uint32_t>(lane % kLanesPerRow) * 16u;
#pragma unroll
  for (int i = 0; i < static_cast<int>(kSub) / kRowsPerInst; ++i) {
    const int row = min(i * kRowsPerInst + rl, nvalid - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&dst[i * kRowsPerInst][0],
                                             16, static_cast<uint32_t>(row) * row_bytes + cb, 0, 0, kStreamCpol);
  }
}

template <typename T>
__device__ __forceinline__ float lds_val(const T (*src)[64], int k, int lane);
template <>
__device__ __forceinline__ float lds_val<float>(const float (*src)[64], int k, int lane) { return src[k][lane]; }
template <>
__device__ __forceinline__ float lds_val<bf16_t>(const bf16_t (*src)[64], int k, int lane) {
  return to_f32(src[k][lane]);
}

// ---------------------------------------------------------------------------
// k_summary state loop: all states of one tile, right to left across tiles.
// f is the tile-local forward state from zero; S accumulates it decayed to the
// chunk end; r is the running reverse state.
//   GEO:  w[k] = exp(delta_k A[d,0]) and abar is its power; B comes from LDS
//         (sB, one row of kSub tokens per state): the state step is short, and
//         the wait of a per-state scalar load would not be hidden.
//   else: w[k] = delta_k and abar = exp2(delta_k A[d,n] log2 e); B comes from
//         the scalar table (bt), which keeps LDS at the two per-lane state
//         arrays; A[d,n] is read one state ahead.
// DS: bit 0 = forward summary (f, S), bit 1 = reverse summary (r, boundary
// states); a one-direction scan computes only what its output pass reads.
// ---------------------------------------------------------------------------
template <int SUB, bool GEO, int DS>
__device__ __forceinline__ void summary_tile_states(int N, int lane, const float (&w)[SUB], const float (&u)[SUB],
                                                    float sigma, float a20, float (*sB)[SUB],
                                                    const float* __restrict__ bt, const float* __restrict__ Arow,
                                                    float (*sR)[64], float (*sS)[64]) {
  float a[SUB];
#pragma unroll
  for (int k = 0; k < SUB; ++k) a[k] = 1.0f;
  float q = 1.0f;
  const float qstep = GEO ? fast_exp2(a20 * sigma) : 1.0f;
  float a2n = GEO ? 0.0f : Arow[0] * kLog2e;
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    const float a2 = a2n;
    if (!GEO) a2n = Arow[min(n + 1, N - 1)] * kLog2e;  // one state ahead
    const sfloat* bn = scalar_ptr(bt + static_cast<size_t>(n) * 2 * SUB);
    float bb[SUB];
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      a[k] = GEO ? a[k] * w[k] : fast_exp2(w[k] * a2);
      bb[k] = u[k] * (GEO ? sB[n][k] : bn[k]);
    }
    // the forward (ascending) and reverse (descending) chains are independent:
    // interleaving them doubles the instruction-level parallelism
    float f = 0.0f;
    float r = (DS & 2) ? sR[n][lane] : 0.0f;
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (DS & 1) f = fmaf(a[t], f, bb[t]);
      if (DS & 2) r = fmaf(a[SUB - 1 - t], r, bb[SUB - 1 - t]);
    }
    if (DS & 1) {
      q = GEO ? q * qstep : fast_exp2(a2 * sigma);
      sS[n][lane] = fmaf(q, f, sS[n][lane]);
    }
    if (DS & 2) sR[n][lane] = r;
  }
}

// ---------------------------------------------------------------------------
// One-direction summary with geometric A: the chunk's end state from zero is a
// sum over its tokens, each input decayed over the tokens between it and the
// chunk edge: S[n] = sum_k rho_k^(n+1) u_k B_k[n], with rho_k = e^(A[d,0] s_k)
// and s_k the sum of delta over those tokens (after k to the chunk end for the
// forward summary, from the chunk start to before k for the reverse one).  So
// rho_k <= 1 and no factor can overflow.  Per state: p_k = u_k rho_k^(n+1) by
// one multiply, then one FMA into S: two operations per (token, channel,
// state) where the recurrence takes three (the power, u B and the chain).
// sAcc[n][lane] accumulates S over the chunk's tiles.
// ---------------------------------------------------------------------------
template <int SUB>
__device__ __forceinline__ void summary_tile_closed(int N, int lane, const float (&rho)[SUB], const float (&u)[SUB],
                                                    float (*sB)[SUB], float (*sAcc)[64]) {
  float p[SUB];
#pragma unroll
  for (int k = 0; k < SUB; ++k) p[k] = u[k];
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    float s0 = sAcc[n][lane], s1 = 0.0f;  // two partial sums: half the dependent chain
#pragma unroll
    for (int k = 0; k < SUB; ++k) p[k] *= rho[k];
#pragma unroll
    for (int k = 0; k < SUB; k += 2) {
      s0 = fmaf(p[k], sB[n][k], s0);
      s1 = fmaf(p[k + 1], sB[n][k + 1], s1);
    }
    sAcc[n][lane] = s0 + s1;
  }
}

// ---------------------------------------------------------------------------
// k_summary: grid (d_inner / 64, nchunk, batch), block 64.  DS as above; P is
// always written (both carries compose with it).  Each wavefront tests its
// channels' A rows and runs the geometric or the general body (a
// wavefront-uniform branch: one launch serves both kinds of channels).
// ---------------------------------------------------------------------------
template <typename T, int NM, bool GEO, int DS>
__device__ __forceinline__ void summary_body(const T* __restrict__ x, const T* __restrict__ dt,
                                             const float* __restrict__ Arow, const float* __restrict__ bct,
                                             const float* __restrict__ dt_bias, int L, int D, int N, int chunk,
                                             int nchunk, int nsub, int ntile, float* __restrict__ Sf,
                                             float* __restrict__ Sr, float* __restrict__ P, float* __restrict__ R,
                                             float* __restrict__ SIG, float (*sR)[64], float (*sS)[64],
                                             float (*sB)[kSub], T (*sX)[64], T (*sDT)[64]) {
  constexpr int SUB = static_cast<int>(kSub);
  // the boundary states feed only an output pass that runs both chains left to right; a
  // reverse-only pass walks right to left and carries its state across tiles instead
  constexpr bool kStoreR = DS == 3;
  const int lane = threadIdx.x;
  const int d = blockIdx.x * 64 + lane;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int t0 = c * chunk;
  const int te = min(L, t0 + chunk);
  const size_t row = static_cast<size_t>(b) * L;
  const size_t cbase = static_cast<size_t>(b) * nchunk + c;
  const float a0 = Arow[0];
  for (int n = 0; n < N; ++n) {
    if (DS & 2) sR[(DS & 2) ? n : 0][lane] = 0.0f;
    if (DS & 1) sS[(DS & 1) ? n : 0][lane] = 0.0f;
  }
  const float a20 = a0 * kLog2e;
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  const uint32_t voff = static_cast<uint32_t>(lane) * IO<T>::kBytes;
  const uint32_t row_bytes = static_cast<uint32_t>(D) * IO<T>::kBytes;
  float sigma = 0.0f;  // sum of delta from the current tile's right edge to the chunk end (kLR: chunk start to its left edge)

  // a one-direction summary with geometric A takes the closed form (summary_tile_closed); the reverse one
  // walks the chunk left to right, so that sigma is the sum of delta before the tile
  constexpr bool kClosed = GEO && DS != 3;
  constexpr bool kLR = kClosed && DS == 2;
  // A one-direction summary brings each tile's x and dt into LDS with direct-to-LDS loads one tile ahead of
  // its walk (its state loop is short, so a tile's loads would otherwise be waited for in full); the pass
  // with both directions loads them straight into registers.
  constexpr bool kPre = DS != 3;
  const int nsub_c = (te - t0 + SUB - 1) / SUB;
  const size_t col0 = static_cast<size_t>(blockIdx.x) * 64;
  if (kPre) {
    const int jf = kLR ? 0 : nsub_c - 1;  // the walk's first tile
    const int tsf = t0 + jf * SUB;
    const int nvf = min(SUB, te - tsf);
    lds_load_tile<T>(x + (row + tsf) * D + col0, nvf, row_bytes, sX, lane);
    lds_load_tile<T>(dt + (row + tsf) * D + col0, nvf, row_bytes, sDT, lane);
  }
  for (int jj = 0; jj < nsub_c; ++jj) {
    const int j = kLR ? jj : nsub_c - 1 - jj;
    const int ts = t0 + j * SUB;
    const int nvalid = min(SUB, te - ts);
    const size_t tile = (row + ts) * D + col0;
    const size_t tile_bytes = static_cast<size_t>(nvalid) * row_bytes;
    float xr[SUB], dr[SUB];
    if (kPre) {
      // this tile's x and dt are in LDS once every vector load issued so far is done
      wait_vmem_all();
#pragma unroll
      for (int k = 0; k < SUB; ++k) {
        xr[k] = lds_val<T>(sX, k, lane);
        dr[k] = lds_val<T>(sDT, k, lane);
      }
      wait_lds_all();  // the reads are done before the buffers are refilled
      if (jj + 1 < nsub_c) {
        const int ts1 = t0 + (kLR ? j + 1 : j - 1) * SUB;
        const int nv1 = min(SUB, te - ts1);
        lds_load_tile<T>(x + (row + ts1) * D + col0, nv1, row_bytes, sX, lane);
        lds_load_tile<T>(dt + (row + ts1) * D + col0, nv1, row_bytes, sDT, lane);
      }
    } else {
      load_col_raw<T, SUB>(make_rsrc(x + tile, tile_bytes), voff, row_bytes, nvalid, xr);
      load_col_raw<T, SUB>(make_rsrc(dt + tile, tile_bytes), voff, row_bytes, nvalid, dr);
    }
    const float* bt = bct + (static_cast<size_t>(b) * ntile + static_cast<size_t>(c) * nsub + j) * N * 2 * SUB;
    if (GEO) {
      // copy the tile's B rows (fp32, from the staged table) into LDS: lane = (state, quarter row).
      // One wavefront per workgroup: its LDS accesses are performed in program order.
      const int n = min(lane / (SUB / 4), N - 1);
      const int part = lane % (SUB / 4);
      const float4 v = *reinterpret_cast<const float4*>(bt + static_cast<size_t>(n) * 2 * SUB + part * 4);
      if (lane < NM * (SUB / 4)) *reinterpret_cast<float4*>(&sB[lane / (SUB / 4)][part * 4]) = v;
    }
    // The previous tile's boundary states and suffix sum are stored here, after this tile's loads are
    // issued: vector memory completes in order, so stores issued before the loads would be waited for
    // with them.
    // The stores are issued on every tile, without a branch (on the walk's first tile, and for states
    // n >= N, they fall outside their resources and are dropped), so the compiler can count them and
    // wait for the loads alone.
    if (kStoreR) {
      const bool have = j < nsub_c - 1;
      const size_t jp = cbase * nsub + (have ? j : 0);  // the slot of the boundary left of tile j + 1
      const __amdgpu_buffer_rsrc_t rr =
          make_rsrc(R + jp * N * D + col0, have ? (static_cast<size_t>(N) * D - col0) * 4 : 0);
#pragma unroll
      for (int n = 0; n < NM; ++n)
        IO<float>::store<kStreamCpol>(sR[(DS & 2) ? n : 0][lane], rr,
                                      (static_cast<uint32_t>(n) * static_cast<uint32_t>(D) + lane) * 4u, 0);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(SIG + jp * D + col0, have ? 256 : 0);
      IO<float>::store<kStreamCpol>(sigma, rs, static_cast<uint32_t>(lane) * 4u, 0);
    }
    float dl[SUB], u[SUB];
    tile_delta<SUB>(dr, bias, nvalid, dl);
    float tile_sum = 0.0f;
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      u[k] = dl[k] * xr[k];
      tile_sum += dl[k];
    }
    if (kClosed) {
      // rho_k = e^(A[d,0] s_k): s_k sums delta from token k (exclusive) to the chunk end, or from the chunk
      // start to token k (exclusive); sigma holds the part outside this tile
      float rho[SUB];
      float run = sigma;
      if (DS == 1) {
#pragma unroll
        for (int k = SUB - 1; k >= 0; --k) {
          rho[k] = fast_exp2(a20 * run);
          run += dl[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
          rho[k] = fast_exp2(a20 * run);
          run += dl[k];
        }
      }
      summary_tile_closed<SUB>(N, lane, rho, u, sB, (DS == 1) ? sS : sR);
    } else if (GEO) {
      float w[SUB];
#pragma unroll
      for (int k = 0; k < SUB; ++k) w[k] = fast_exp2(dl[k] * a20);
      summary_tile_states<SUB, true, DS>(N, lane, w, u, sigma, a20, sB, bt, Arow, sR, sS);
    } else {
      summary_tile_states<SUB, false, DS>(N, lane, dl, u, sigma, a20, sB, bt, Arow, sR, sS);
    }
    sigma += tile_sum;
  }
  for (int n = 0; n < N; ++n) {
    const size_t o = (cbase * N + n) * D + d;
    if (DS & 1) Sf[o] = sS[(DS & 1) ? n : 0][lane];
    if (DS & 2) Sr[o] = sR[(DS & 2) ? n : 0][lane];
    P[o] = fast_exp2(Arow[n] * kLog2e * sigma);
  }
}

template <typename T, int NM, int DS>
__global__ __launch_bounds__(64) void k_summary(const T* __restrict__ x, const T* __restrict__ dt,
                                                const float* __restrict__ A, const float* __restrict__ bct,
                                                const float* __restrict__ dt_bias, int L, int D, int N, int chunk,
                                                int nchunk, int nsub, int ntile, float* __restrict__ Sf,
                                                float* __restrict__ Sr, float* __restrict__ P,
                                                float* __restrict__ R, float* __restrict__ SIG) {
  static_assert(NM * static_cast<int>(kSub) <= 64 * 4, "one float4 of B per lane");
  __shared__ float sR[(DS & 2) ? NM : 1][64];
  __shared__ float sS[(DS & 1) ? NM : 1][64];
  __shared__ __align__(16) float sB[NM][kSub];  // the tile's B, one row per state (geometric body)
  __shared__ __align__(16) T sX[(DS != 3) ? kSub : 1][64];  // a one-direction pass's next x and dt tiles
  __shared__ __align__(16) T sDT[(DS != 3) ? kSub : 1][64];
  const int d = blockIdx.x * 64 + threadIdx.x;
  const float* __restrict__ Arow = A + static_cast<size_t>(d) * N;
  const float a0 = Arow[0];
  bool geo_lane = true;
  for (int n = 0; n < N; ++n) geo_lane = geo_lane && (Arow[n] == static_cast<float>(n + 1) * a0);
  if (wave_geometric(geo_lane)) {
    summary_body<T, NM, true, DS>(x, dt, Arow, bct, dt_bias, L, D, N, chunk, nchunk, nsub, ntile, Sf, Sr, P, R, SIG,
                                  sR, sS, sB, sX, sDT);
  } else {
    summary_body<T, NM, false, DS>(x, dt, Arow, bct, dt_bias, L, D, N, chunk, nchunk, nsub, ntile, Sf, Sr, P, R,
                                   SIG, sR, sS, sB, sX, sDT);
  }
}

// ---------------------------------------------------------------------------
// k_carry: one thread per (b, n, d); sequential over chunks in both directions.
// The two directions run in one loop (two independent chains), and the inputs
// of kBatch chunks are loaded before they are composed, so the loop pays one
// memory latency per batch rather than one per chunk.
// ---------------------------------------------------------------------------
// The batch-0 threads also write the transposed table A2T[n][d] = A[d,n] * log2(e)
// that the output pass reads with coalesced loads.
__global__ __launch_bounds__(256) void k_carry(const float* __restrict__ Sf, const float* __restrict__ Sr,
                                               const float* __restrict__ P, float* __restrict__ Cf,
                                               float* __restrict__ Cr, const float* __restrict__ h_in,
                                               const float* __restrict__ A, float* __restrict__ A2T, int batch,
                                               int nchunk, int N, int D) {
  constexpr int kBatch = 16;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t total = static_cast<size_t>(batch) * N * D;
  if (idx >= total) return;
  const int d = static_cast<int>(idx % D);
  const int n = static_cast<int>((idx / D) % N);
  const int b = static_cast<int>(idx / (static_cast<size_t>(D) * N));
  if (b == 0) A2T[static_cast<size_t>(n) * D + d] = A[static_cast<size_t>(d) * N + n] * kLog2e;
  const size_t base = (static_cast<size_t>(b) * nchunk * N + n) * D + d;  // chunk 0
  const size_t stride = static_cast<size_t>(N) * D;                       // per chunk
  float cf = h_in ? h_in[(static_cast<size_t>(b) * D + d) * N + n] : 0.0f;
  float cr = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += kBatch) {
    float pf[kBatch], sf[kBatch], pr[kBatch], sr[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const size_t of = base + static_cast<size_t>(min(c0 + i, nchunk - 1)) * stride;            // forward: c0 + i
      const size_t orr = base + static_cast<size_t>(max(nchunk - 1 - c0 - i, 0)) * stride;      // reverse
      pf[i] = P[of];
      sf[i] = Sf[of];
      pr[i] = P[orr];
      sr[i] = Sr[orr];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i < nchunk) {
        Cf[base + static_cast<size_t>(c0 + i) * stride] = cf;
        cf = fmaf(pf[i], cf, sf[i]);
        Cr[base + static_cast<size_t>(nchunk - 1 - c0 - i) * stride] = cr;
        cr = fmaf(pr[i], cr, sr[i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_output state loop: all states of one tile.  GEO: w[k] = exp(delta_k A[d,0])
// and abar is its power; otherwise w[k] = delta_k.
// DIRS: bit 0 = forward readout, bit 1 = reverse readout.
//
// The reverse state entering the tile from the right is formed per state from
// the zero-started boundary state Rj[n] (summary pass) and the chunk's carry
// Cr[n]: hr = Rj[n] + exp(A[d,n] sigma_j) Cr[n], sigma_j being the sum of delta
// from the tile's right edge to the chunk end (on the chunk's last tile, hr =
// Cr[n]).  Rj, Cr and (general A) A[d,n] log2(e) are read with vector loads one
// state ahead; vector loads complete in order, so only the oldest is waited for.
// ---------------------------------------------------------------------------
template <int SUB, int DIRS, bool GEO>
__device__ __forceinline__ void output_tile_states(int N, int D, int lane, const float (&w)[SUB],
                                                   const float (&u)[SUB], float (&y)[SUB],
                                                   const float* __restrict__ bt, float (*sHf)[64],
                                                   __amdgpu_buffer_rsrc_t rj_rsrc, __amdgpu_buffer_rsrc_t cr_rsrc,
                                                   __amdgpu_buffer_rsrc_t a2_rsrc, float qstep, float sj,
                                                   bool last, bool keep_hf) {
  constexpr bool kRev = (DIRS & 2) != 0;
  constexpr bool kSum = DIRS == 3;
  // the forward chain runs for the forward readout or for the cached forward state
  const bool fwd_chain = (DIRS & 1) != 0 || keep_hf;
  const uint32_t voff4 = static_cast<uint32_t>(lane) * 4u;
  const uint32_t nstride4 = static_cast<uint32_t>(D) * 4u;
  float a[SUB];
#pragma unroll
  for (int k = 0; k < SUB; ++k) a[k] = 1.0f;
  float q = 1.0f;
  float rj_next = 0.0f, cr_next = 0.0f, a2_next = 0.0f;
  if (kRev) {
    rj_next = IO<float>::load<kStreamCpol>(rj_rsrc, voff4, 0);
    cr_next = IO<float>::load(cr_rsrc, voff4, 0);
  }
  if (!GEO) a2_next = IO<float>::load(a2_rsrc, voff4, 0);
  if constexpr (DIRS == 1) {
    // Forward readout only: every u B product is formed before the chain, so B's uses all precede C's, and
    // each half of the state's table row is loaded half a state ahead into registers whose values are dead:
    // C of state n after the first use of B, B of state n + 1 after the first use of C.  Scalar loads
    // complete out of order (a wait for one waits for all issued before it), so this order keeps each wait
    // from covering a load issued just before it.  The scheduling barriers hold the loads in place.
    float bv[SUB], cv[SUB];
    float hf_next = sHf[0][lane];
    {
      const sfloat* b0 = scalar_ptr(bt);
#pragma unroll
      for (int k = 0; k < SUB; ++k) bv[k] = b0[k];
    }
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
      const sfloat* cn = scalar_ptr(bt + static_cast<size_t>(n) * 2 * SUB + SUB);
      const sfloat* bn1 = scalar_ptr(bt + static_cast<size_t>(min(n + 1, N - 1)) * 2 * SUB);
      float a2 = 0.0f;
      if (!GEO) {
        a2 = a2_next;
        a2_next = IO<float>::load(a2_rsrc, voff4, static_cast<uint32_t>(min(n + 1, N - 1)) * nstride4);
      }
      float hf = hf_next;
      float bb[SUB];
      a[0] = GEO ? a[0] * w[0] : fast_exp2(w[0] * a2);
      bb[0] = u[0] * bv[0];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < SUB; ++k) cv[k] = cn[k];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 1; k < SUB; ++k) {
        a[k] = GEO ? a[k] * w[k] : fast_exp2(w[k] * a2);
        bb[k] = u[k] * bv[k];
      }
      hf = fmaf(a[0], hf, bb[0]);
      y[0] = fmaf(cv[0], hf, y[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < SUB; ++k) bv[k] = bn1[k];
      hf_next = sHf[min(n + 1, N - 1)][lane];  // sHf[n + 1] is not written in this step
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 1; k < SUB; ++k) {
        hf = fmaf(a[k], hf, bb[k]);
        y[k] = fmaf(cv[k], hf, y[k]);
      }
      sHf[n][lane] = hf;
    }
    return;
  }
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    const sfloat* bn = scalar_ptr(bt + static_cast<size_t>(n) * 2 * SUB);
    const uint32_t s1 = static_cast<uint32_t>(min(n + 1, N - 1)) * nstride4;
    float a2 = 0.0f;
    if (!GEO) {
      a2 = a2_next;
      a2_next = IO<float>::load(a2_rsrc, voff4, s1);
    }
    float hf = fwd_chain ? sHf[n][lane] : 0.0f;
    float rj = 0.0f, cr = 0.0f;
    if (kRev) {
      rj = rj_next;
      cr = cr_next;
      rj_next = IO<float>::load<kStreamCpol>(rj_rsrc, voff4, s1);
      cr_next = IO<float>::load(cr_rsrc, voff4, s1);
    }
    float bb[SUB];
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      a[k] = GEO ? a[k] * w[k] : fast_exp2(w[k] * a2);
      bb[k] = u[k] * bn[k];
    }
    float hk[kSum ? SUB : 1];  // with both readouts: the forward state after token k
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      if (fwd_chain) hf = fmaf(a[k], hf, bb[k]);
      if (kSum) hk[kSum ? k : 0] = hf;
      else if (DIRS & 1) y[k] = fmaf(bn[SUB + k], hf, y[k]);
    }
    if (kRev) {
      q = GEO ? q * qstep : fast_exp2(a2 * sj);
      // the last tile's boundary slot is never written: its value is discarded here
      float hr = last ? cr : fmaf(q, cr, rj);
#pragma unroll
      for (int k = SUB - 1; k >= 0; --k) {
        hr = fmaf(a[k], hr, bb[k]);
        // both readouts share one product with C_t[n]: C . h_fwd + C . h_rev = C . (h_fwd + h_rev)
        y[k] = fmaf(bn[SUB + k], kSum ? hr + hk[kSum ? k : 0] : hr, y[k]);
      }
    }
    if (fwd_chain) sHf[n][lane] = hf;
  }
}

// ---------------------------------------------------------------------------
// k_output state loop of the right-to-left walk (reverse readout only): the
// reverse state of each state index is carried across the chunk's tiles in sH,
// starting from the chunk's carry from the right, so no boundary state is read.
// ---------------------------------------------------------------------------
template <int SUB, bool GEO>
__device__ __forceinline__ void output_tile_states_rwalk(int N, int D, int lane, const float (&w)[SUB],
                                                         const float (&u)[SUB], float (&y)[SUB],
                                                         const float* __restrict__ bt, float (*sH)[64],
                                                         __amdgpu_buffer_rsrc_t a2_rsrc) {
  const uint32_t voff4 = static_cast<uint32_t>(lane) * 4u;
  const uint32_t nstride4 = static_cast<uint32_t>(D) * 4u;
  float a[SUB];
#pragma unroll
  for (int k = 0; k < SUB; ++k) a[k] = 1.0f;
  float a2_next = GEO ? 0.0f : IO<float>::load(a2_rsrc, voff4, 0);
  // B's uses all precede C's in a state step: each half of the state's table row is loaded half a state
  // ahead into registers whose values are dead, as in the forward-only readout of output_tile_states
  float bv[SUB], cv[SUB];
  float hr_next = sH[0][lane];
  {
    const sfloat* b0 = scalar_ptr(bt);
#pragma unroll
    for (int k = 0; k < SUB; ++k) bv[k] = b0[k];
  }
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    const sfloat* cn = scalar_ptr(bt + static_cast<size_t>(n) * 2 * SUB + SUB);
    const sfloat* bn1 = scalar_ptr(bt + static_cast<size_t>(min(n + 1, N - 1)) * 2 * SUB);
    float a2 = 0.0f;
    if (!GEO) {
      a2 = a2_next;
      a2_next = IO<float>::load(a2_rsrc, voff4, static_cast<uint32_t>(min(n + 1, N - 1)) * nstride4);
    }
    float hr = hr_next;
    float bb[SUB];
    a[0] = GEO ? a[0] * w[0] : fast_exp2(w[0] * a2);
    bb[0] = u[0] * bv[0];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < SUB; ++k) cv[k] = cn[k];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 1; k < SUB; ++k) {
      a[k] = GEO ? a[k] * w[k] : fast_exp2(w[k] * a2);
      bb[k] = u[k] * bv[k];
    }
    {
      constexpr int k = SUB - 1;
      hr = fmaf(a[k], hr, bb[k]);
      y[k] = fmaf(cv[k], hr, y[k]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < SUB; ++k) bv[k] = bn1[k];
    hr_next = sH[min(n + 1, N - 1)][lane];  // sH[n + 1] is not written in this step
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = SUB - 2; k >= 0; --k) {
      hr = fmaf(a[k], hr, bb[k]);
      y[k] = fmaf(cv[k], hr, y[k]);
    }
    sH[n][lane] = hr;
  }
}

// ---------------------------------------------------------------------------
// k_output: grid (d_inner / 64, nchunk, batch), block 64 (one wavefront).
// x, dt and z tiles are brought into LDS one tile ahead with direct-to-LDS
// loads, so the HBM stream of tile j+1 overlaps the state loop of tile j (all
// wavefronts run the same loop in step; without this they would all wait for
// memory at the same time and then all compute).
// ---------------------------------------------------------------------------
template <typename T, int DIRS, bool GEO>
__device__ __forceinline__ void output_body(const T* __restrict__ x, const T* __restrict__ dt,
                                            const T* __restrict__ z, float a0, const float* __restrict__ bct,
                                            const float* __restrict__ Dv, const float* __restrict__ dt_bias,
                                            T* __restrict__ out, int L, int D, int N, int chunk, int nchunk, int nsub,
                                            int ntile, int gate, const float* __restrict__ Cf,
                                            const float* __restrict__ Cr, const float* __restrict__ R,
                                            const float* __restrict__ SIG, const float* __restrict__ A2T,
                                            float* __restrict__ h_out, float (*sHf)[64], T (*sX)[64], T (*sDT)[64],
                                            T (*sZ)[64]) {
  constexpr int SUB = static_cast<int>(kSub);
  // DIRS bit 2: reverse readout only, tiles walked right to left with the reverse state carried
  constexpr bool kRW = (DIRS & 4) != 0;
  constexpr int DR = DIRS & 3;  // the readouts
  const int lane = threadIdx.x;
  const int d = blockIdx.x * 64 + lane;
  const size_t col0 = static_cast<size_t>(blockIdx.x) * 64;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int t0 = c * chunk;
  const int te = min(L, t0 + chunk);
  const size_t row = static_cast<size_t>(b) * L;
  const size_t cbase = static_cast<size_t>(b) * nchunk + c;
  for (int n = 0; n < N; ++n) sHf[n][lane] = (kRW ? Cr : Cf)[(cbase * N + n) * D + d];
  const float a20 = a0 * kLog2e;
  const float bias = dt_bias ? dt_bias[d] : 0.0f;
  constexpr float ndir = (DR == 3) ? 2.0f : 1.0f;
  const float skip = Dv ? ndir * Dv[d] : 0.0f;
  const uint32_t voff = static_cast<uint32_t>(lane) * IO<T>::kBytes;
  const uint32_t row_bytes = static_cast<uint32_t>(D) * IO<T>::kBytes;
  const size_t state_bytes = static_cast<size_t>(N) * D * 4;
  const __amdgpu_buffer_rsrc_t cr_rsrc = make_rsrc(Cr + cbase * N * D + col0, state_bytes);
  const __amdgpu_buffer_rsrc_t a2_rsrc = make_rsrc(A2T + col0, state_bytes);

  const int nsub_c = (te - t0 + SUB - 1) / SUB;
  {
    const int tf = t0 + (kRW ? nsub_c - 1 : 0) * SUB;  // the first tile of the walk
    const size_t tile = (row + tf) * D + col0;
    const int nv = min(SUB, te - tf);
    lds_load_tile<T>(x + tile, nv, row_bytes, sX, lane);
    lds_load_tile<T>(dt + tile, nv, row_bytes, sDT, lane);
    if (gate) lds_load_tile<T>(z + tile, nv, row_bytes, sZ, lane);
  }
  for (int jj = 0; jj < nsub_c; ++jj) {
    const int j = kRW ? nsub_c - 1 - jj : jj;
    const int ts = t0 + j * SUB;
    const int nvalid = min(SUB, te - ts);
    const bool last = (jj == nsub_c - 1);  // the last tile of the walk: nothing to prefetch
    const int ts1 = ts + (kRW ? -SUB : SUB);  // the next tile of the walk
    const size_t jb = cbase * nsub + j;
    const size_t tile = (row + ts) * D + col0;
    const size_t tile_bytes = static_cast<size_t>(nvalid) * row_bytes;
    // this tile's x and dt are in LDS once every vector load issued so far is done
    wait_vmem_all();
    float xr[SUB], dr[SUB];
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      xr[k] = lds_val<T>(sX, k, lane);
      dr[k] = lds_val<T>(sDT, k, lane);
    }
    wait_lds_all();  // the reads are done before the buffers are refilled
    if (!last) {
      const size_t tile1 = (row + ts1) * D + col0;
      const int nv1 = min(SUB, te - ts1);
      lds_load_tile<T>(x + tile1, nv1, row_bytes, sX, lane);
      lds_load_tile<T>(dt + tile1, nv1, row_bytes, sDT, lane);
    }
    // the left-to-right walk's reverse chain enters each tile from its stored boundary state
    const bool chunk_end = (j == nsub_c - 1);
    const float sj = (kRW || chunk_end || !(DR & 2)) ? 0.0f : __builtin_nontemporal_load(&SIG[jb * D + d]);
    const float* bt = bct + (static_cast<size_t>(b) * ntile + static_cast<size_t>(c) * nsub + j) * N * 2 * SUB;
    const __amdgpu_buffer_rsrc_t rj_rsrc = make_rsrc(R + jb * N * D + col0, state_bytes);
    float dl[SUB], u[SUB], y[SUB];
    tile_delta<SUB>(dr, bias, nvalid, dl);
#pragma unroll
    for (int k = 0; k < SUB; ++k) {
      u[k] = dl[k] * xr[k];
      y[k] = skip * xr[k];
    }
    if (kRW) {
      if (GEO) {
        float w[SUB];
#pragma unroll
        for (int k = 0; k < SUB; ++k) w[k] = fast_exp2(dl[k] * a20);
        output_tile_states_rwalk<SUB, true>(N, D, lane, w, u, y, bt, sHf, a2_rsrc);
      } else {
        output_tile_states_rwalk<SUB, false>(N, D, lane, dl, u, y, bt, sHf, a2_rsrc);
      }
    } else if (GEO) {
      float w[SUB];
#pragma unroll
      for (int k = 0; k < SUB; ++k) w[k] = fast_exp2(dl[k] * a20);
      output_tile_states<SUB, DR, true>(N, D, lane, w, u, y, bt, sHf, rj_rsrc, cr_rsrc, a2_rsrc,
                                        fast_exp2(a20 * sj), sj, chunk_end, h_out != nullptr);
    } else {
      output_tile_states<SUB, DR, false>(N, D, lane, dl, u, y, bt, sHf, rj_rsrc, cr_rsrc, a2_rsrc, 1.0f, sj,
                                         chunk_end, h_out != nullptr);
    }
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + tile, tile_bytes);
    if (gate) {
      wait_vmem_all();  // this tile's z
      float zr[SUB];
#pragma unroll
      for (int k = 0; k < SUB; ++k) zr[k] = lds_val<T>(sZ, k, lane);
      wait_lds_all();
      if (!last) lds_load_tile<T>(z + (row + ts1) * D + col0, min(SUB, te - ts1), row_bytes, sZ, lane);
#pragma unroll
      for (int k = 0; k < SUB; ++k) y[k] *= silu_f32(zr[k]);
    }
    store_col<T, SUB>(y, ro, voff, row_bytes, nvalid);
  }
  if (!kRW && h_out != nullptr && c == nchunk - 1) {
    for (int n = 0; n < N; ++n) h_out[(static_cast<size_t>(b) * D + d) * N + n] = sHf[n][lane];
  }
}

template <typename T, int NM, int DIRS>
__global__ __launch_bounds__(64) void k_output(const T* __restrict__ x, const T* __restrict__ dt,
                                               const T* __restrict__ z, const float* __restrict__ A,
                                               const float* __restrict__ bct, const float* __restrict__ Dv,
                                               const float* __restrict__ dt_bias, T* __restrict__ out, int L, int D,
                                               int N, int chunk, int nchunk, int nsub, int ntile, int gate,
                                               const float* __restrict__ Cf, const float* __restrict__ Cr,
                                               const float* __restrict__ R, const float* __restrict__ SIG,
                                               const float* __restrict__ A2T, float* __restrict__ h_out) {
  __shared__ float sHf[NM][64];  // per-lane carried state (forward, or reverse for a right-to-left walk)
  __shared__ __align__(16) T sX[kSub][64];
  __shared__ __align__(16) T sDT[kSub][64];
  __shared__ __align__(16) T sZ[kSub][64];
  const int d = blockIdx.x * 64 + threadIdx.x;
  const float* __restrict__ Arow = A + static_cast<size_t>(d) * N;
  const float a0 = Arow[0];
  bool geo_lane = true;
  for (int n = 0; n < N; ++n) geo_lane = geo_lane && (Arow[n] == static_cast<float>(n + 1) * a0);
  if (wave_geometric(geo_lane)) {
    output_body<T, DIRS, true>(x, dt, z, a0, bct, Dv, dt_bias, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf, Cr,
                               R, SIG, A2T, h_out, sHf, sX, sDT, sZ);
  } else {
    output_body<T, DIRS, false>(x, dt, z, a0, bct, Dv, dt_bias, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf,
                                Cr, R, SIG, A2T, h_out, sHf, sX, sDT, sZ);
  }
}

// ---------------------------------------------------------------------------
// k_block: one short block of block-cache decoding in a single kernel (the
// forward direction from the cached state, the reverse direction from zero at
// the block's last token; the new cache is the forward state after the block).
// grid (d_inner / 16, batch), block 256 HV (HV groups of four wavefronts).  A
// workgroup owns 16 channels and every state of them: lane l of wavefront w of
// a group runs channel 16 blockIdx.x + l / 4 and state 4 w + l % 4, so the
// 16 x 16 recurrences of a workgroup run side by side, one per lane, and a
// block step fills the chip (d_inner / 16 workgroups).  The block is padded to
// GM tokens (GM in {16, 32, 64, 128}); padding tokens have delta = 0 and no
// input, so they leave every state unchanged and are never stored.  With
// HV = 2 (GM >= 32) the two halves of the block run side by side, one per
// group, so each recurrence walks GM / 2 tokens at a time:
//   first half: forward chain from the cache   | second half: reverse chain from zero
//   (both leave their state at the halves' boundary in LDS; barrier)
//   first half: reverse chain from the second  | second half: forward chain from the
//   half's boundary state                      | first half's end state; the new cache
// Each chain is exact: it starts from the state that enters its half.
//   1. every global load of the kernel is issued at once, from clamped in-bounds
//      addresses: the lane's A[d,n] and cached state, and per (token, channel)
//      dt, x, z, and B, C; delta, delta*x, the skip term D*x and the gate SiLU(z)
//      go to LDS, B and C (fp32) too;
//   2. each lane: abar and delta*x*B per token of its half in registers, the two
//      chains as above with the state per token kept, and C_t[n] (h_fwd + h_rev)
//      per token; the four states of a channel in a wavefront are summed across
//      the lane quad (DPP), the four wavefronts' sums meet in LDS and are added
//      in a fixed order (deterministic);
//   3. skip term, gate, store.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld_any(const T* p);
template <>
__device__ __forceinline__ float ld_any<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_any<bf16_t>(const bf16_t* p) { return to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st_any(T* p, float v);
template <>
__device__ __forceinline__ void st_any<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st_any<bf16_t>(bf16_t* p, float v) {
  const __bf16 h = static_cast<__bf16>(v);  // round to nearest even
  p->bits = __builtin_bit_cast(unsigned short, h);
}

template <int GM, int HV>
struct BlockSmem {
  static constexpr int kRow = GM + 4;  // B and C rows padded: the four states a wavefront reads sit in different banks
  float dl[GM][16];
  float u[GM][16];
  float sx[GM][16];  // skip * x
  float g[GM][16];   // SiLU(z), or 1 without the gate
  __attribute__((aligned(16))) float b[16][kRow];
  __attribute__((aligned(16))) float c[16][kRow];
  float part[4][GM][16];
  float edge[HV][HV == 2 ? 16 : 1][16];  // two halves: [fwd, rev][state][channel] at the halves' boundary
};

// sum over the lane quad (the four states of a channel): lanes (0+1) + (2+3) in every quad
__device__ __forceinline__ float quad_sum(float v) {
  constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // quad_perm [1, 0, 3, 2]
  constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // quad_perm [2, 3, 0, 1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kXor1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kXor2, 0xf, 0xf, false));
  return v;
}

// Step 1 of the block kernels.  Every global load is issued at once, from clamped in-bounds addresses (a load
// under a branch is waited for at the branch's end), and the values are selected afterwards; stand-ins for
// absent tensors: A for h_in, D and dt_bias, x for z (their values are not used).  Then delta, delta * x, the
// skip term D x (counted once per direction the output keeps) and the gate SiLU(z) per (token, channel), and
// B, C per (state, token), go to LDS, zero past the block and for states n >= N.  Returns the lane's A[d, n]
// and cached state (read before any write: h_out may alias h_in, and every write of h_out follows a barrier
// after this).  The caller synchronises before reading the LDS.
template <typename T, int GM, int kThreads, typename SM>
__device__ __forceinline__ void block_stage(SM& sm, const T* __restrict__ x, const T* __restrict__ dt,
                                            const T* __restrict__ z, const float* __restrict__ A,
                                            const T* __restrict__ Bm, const T* __restrict__ Cm,
                                            const float* __restrict__ Dv, const float* __restrict__ dt_bias,
                                            const float* h_in, int G, int D, int N, bool gate, bool both, int n,
                                            int d, int b, float& av, float& hv) {
  // (token, channel) pairs, and B, C elements, per thread: GM * 16 of each over kThreads threads (with more
  // threads than pairs, the threads past them only load clamped stand-ins and store nothing)
  constexpr int kPairs = GM * 16;
  constexpr int kTpt = (kPairs + kThreads - 1) / kThreads;
  constexpr bool kAll = kPairs % kThreads == 0;
  const int tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * G;  // first token row of this batch element
  const int nc = min(n, N - 1);
  av = A[static_cast<size_t>(d) * N + nc];
  const size_t hs = h_in ? (static_cast<size_t>(b) * D + d) * N + nc : static_cast<size_t>(d) * N + nc;
  hv = (h_in ? h_in : A)[hs];
  const int c1 = tid & 15;  // channel of this thread's (token, channel) pairs
  const int d1 = blockIdx.x * 16 + c1;
  const float dvv = (Dv ? Dv : A)[d1];
  const float bsv = (dt_bias ? dt_bias : A)[d1];
  const T* zbase = gate ? z : x;
  float xv[kTpt], dv[kTpt], zv[kTpt], bv[kTpt], cv[kTpt];
#pragma unroll
  for (int k = 0; k < kTpt; ++k) {
    const int i = min(tid + kThreads * k, kPairs - 1);  // pair (token i / 16, channel i % 16); B, C element
    const int t = i / 16;                               // (state i / GM, token i % GM)
    const size_t o = (row + min(t, G - 1)) * D + d1;
    xv[k] = ld_any(x + o);
    dv[k] = ld_any(dt + o);
    zv[k] = ld_any(zbase + o);
    const size_t ob = (row + min(i % GM, G - 1)) * N + min(i / GM, N - 1);
    bv[k] = ld_any(Bm + ob);
    cv[k] = ld_any(Cm + ob);
  }
  const float bias = dt_bias ? bsv : 0.0f;
  const float skip = Dv ? (both ? 2.0f : 1.0f) * dvv : 0.0f;
#pragma unroll
  for (int k = 0; k < kTpt; ++k) {
    const int i = tid + kThreads * k;
    if (!kAll && i >= kPairs) break;
    const int t = i / 16;
    const bool live = t < G;
    const float dl = live ? softplus_f32(dv[k] + bias) : 0.0f;
    const float xl = live ? xv[k] : 0.0f;
    sm.dl[t][c1] = dl;
    sm.u[t][c1] = dl * xl;
    sm.sx[t][c1] = skip * xl;
    sm.g[t][c1] = (live && gate) ? silu_f32(zv[k]) : 1.0f;
    const bool ok = i / GM < N && i % GM < G;
    sm.b[i / GM][i % GM] = ok ? bv[k] : 0.0f;
    sm.c[i / GM][i % GM] = ok ? cv[k] : 0.0f;
  }
}

// Step 3 of the block kernels: the four wavefronts' sums of a token (in sm.part) in a fixed order, the skip
// term and the gate, and the store.
template <typename T, int GM, int kThreads, typename SM>
__device__ __forceinline__ void block_store(const SM& sm, T* __restrict__ out, int G, int D, int b) {
  constexpr int kPairs = GM * 16;
  constexpr int kTpt = (kPairs + kThreads - 1) / kThreads;
  const int tid = threadIdx.x, c1 = tid & 15;
  const int d1 = blockIdx.x * 16 + c1;
  const size_t row = static_cast<size_t>(b) * G;
#pragma unroll
  for (int k = 0; k < kTpt; ++k) {
    const int i = tid + kThreads * k;
    const int t = i / 16;
    if (i < kPairs && t < G) {
      const float acc = ((sm.part[0][t][c1] + sm.part[1][t][c1]) + sm.part[2][t][c1]) + sm.part[3][t][c1];
      st_any(out + (row + t) * D + d1, (acc + sm.sx[t][c1]) * sm.g[t][c1]);
    }
  }
}

template <typename T, int GM, int HV>
__global__ __launch_bounds__(256 * HV) void k_block(const T* __restrict__ x, const T* __restrict__ dt,
                                                    const T* __restrict__ z, const float* __restrict__ A,
                                                    const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                    const float* __restrict__ Dv, const float* __restrict__ dt_bias,
                                                    const float* h_in, float* h_out, T* __restrict__ out, int G,
                                                    int D, int N, int flags) {
  using S = BlockSmem<GM, HV>;
  static_assert(HV == 1 || (HV == 2 && GM >= 32), "halves of at least 16 tokens");
  constexpr int kThreads = 256 * HV;
  constexpr int GH = GM / HV;  // tokens per half
  __shared__ S sm;
  const int tid = threadIdx.x;
  const int half = HV == 2 ? tid / 256 : 0;  // wavefront-uniform
  const int wv = (tid % 256) / 64;
  const int lane = tid % 64;
  const int cl = lane >> 2;           // channel of this lane's recurrence, within the workgroup
  const int n = wv * 4 + (lane & 3);  // its state
  const int d = blockIdx.x * 16 + cl;
  const int b = blockIdx.y;
  const bool gate = (flags & kNoGate) == 0;
  const bool fwd = (flags & kRevOnly) == 0;
  const bool rev = (flags & kFwdOnly) == 0;

  // 1. loads and LDS staging
  float av, hv;
  block_stage<T, GM, kThreads>(sm, x, dt, z, A, Bm, Cm, Dv, dt_bias, h_in, G, D, N, gate, fwd && rev, n, d, b, av,
                               hv);
  __syncthreads();

  // 2. this lane's recurrences over the tokens t0 .. t0 + GH - 1 of its half (states n >= N have
  //    B = C = 0: they stay 0 and add nothing)
  const int t0 = half * GH;
  const float a2 = n < N ? av * kLog2e : 0.0f;
  float a[GH], bb[GH], y[GH];
#pragma unroll
  for (int t4 = 0; t4 < GH / 4; ++t4) {
    const float4 bq = *reinterpret_cast<const float4*>(&sm.b[n][t0 + 4 * t4]);
    const float bq4[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * t4 + i;
      a[t] = fast_exp2(sm.dl[t0 + t][cl] * a2);
      bb[t] = sm.u[t0 + t][cl] * bq4[i];
    }
  }
  if (half == 0) {
    // the forward chain from the cache; its state per token is kept in y
    float hf = (n < N && h_in) ? hv : 0.0f;
#pragma unroll
    for (int t = 0; t < GH; ++t) {
      hf = fmaf(a[t], hf, bb[t]);
      y[t] = fwd ? hf : 0.0f;
    }
    if (HV == 1) {
      if (h_out && n < N) h_out[(static_cast<size_t>(b) * D + d) * N + n] = hf;  // padding leaves hf unchanged
    } else {
      sm.edge[0][HV == 2 ? n : 0][cl] = hf;
    }
  } else {
    // second half: the reverse chain from zero at the block's last token
    float hr = 0.0f;
#pragma unroll
    for (int t = GH - 1; t >= 0; --t) {
      hr = fmaf(a[t], hr, bb[t]);
      y[t] = rev ? hr : 0.0f;
    }
    sm.edge[HV == 2 ? 1 : 0][HV == 2 ? n : 0][cl] = hr;
  }
  if (HV == 2) __syncthreads();
  if (half == 0) {
    // the reverse chain, entering the first half from the second (zero with one half)
    float hr = HV == 2 ? sm.edge[HV == 2 ? 1 : 0][HV == 2 ? n : 0][cl] : 0.0f;
#pragma unroll
    for (int t4 = GH / 4 - 1; t4 >= 0; --t4) {
      const float4 cq = *reinterpret_cast<const float4*>(&sm.c[n][t0 + 4 * t4]);
      const float cq4[4] = {cq.x, cq.y, cq.z, cq.w};
      // with two halves, delta*x*B is formed again here rather than held across the barrier
      const float4 bq = HV == 2 ? *reinterpret_cast<const float4*>(&sm.b[n][t0 + 4 * t4]) : cq;
      const float bq4[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const int t = 4 * t4 + i;
        if (rev) {
          hr = fmaf(a[t], hr, HV == 2 ? sm.u[t0 + t][cl] * bq4[i] : bb[t]);
          y[t] += hr;
        }
        y[t] = quad_sum(y[t] * cq4[i]);
      }
    }
  } else {
    // second half: the forward chain from the first half's end state; the new cache
    float hf = sm.edge[0][HV == 2 ? n : 0][cl];
#pragma unroll
    for (int t4 = 0; t4 < GH / 4; ++t4) {
      const float4 cq = *reinterpret_cast<const float4*>(&sm.c[n][t0 + 4 * t4]);
      const float cq4[4] = {cq.x, cq.y, cq.z, cq.w};
      const float4 bq = *reinterpret_cast<const float4*>(&sm.b[n][t0 + 4 * t4]);
      const float bq4[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * t4 + i;
        hf = fmaf(a[t], hf, sm.u[t0 + t][cl] * bq4[i]);
        if (fwd) y[t] += hf;
        y[t] = quad_sum(y[t] * cq4[i]);
      }
    }
    if (h_out && n < N) h_out[(static_cast<size_t>(b) * D + d) * N + n] = hf;  // padding leaves hf unchanged
  }
  if ((lane & 3) == 0) {
#pragma unroll
    for (int t = 0; t < GH; ++t) sm.part[wv][t0 + t][cl] = y[t];
  }
  __syncthreads();

  // 3. the four wavefronts' sums in a fixed order; skip term, gate, store
  block_store<T, GM, kThreads>(sm, out, G, D, b);
}

// ---------------------------------------------------------------------------
// k_block_parts: the block step with the block cut into NQ parts of GP = GM / NQ tokens, one group of four
// wavefronts per part (lane l of wavefront w of a group: channel 16 blockIdx.x + l / 4, state 4 w + l % 4, as
// in k_block).  A linear recurrence started from zero at a part's edge differs from the true one by the
// entering state carried through the part's decay, so a token's two states are
//   h_fwd(t) = hf(t) + (abar_t0 ... abar_t) h_fwd_in,   h_rev(t) = hr(t) + (abar_t ... abar_t1) h_rev_in
// with hf, hr the part-local chains (t0, t1 the part's first and last token).  Phase 1 runs both local chains
// and the two running products (chains of GP tokens, side by side), keeps C_t (hf + hr) and the two products
// times C_t per token, and leaves the part's product and end states in LDS.  Phase 2 forms the entering
// states from the parts before (forward, from the cache) and after (reverse, from zero) and adds the two
// corrections per token: no chain.  The last part's lanes write the new cache.
// ---------------------------------------------------------------------------
template <int GM, int NQ>
struct BlockSmemParts {
  static constexpr int kRow = GM + 4;  // B and C rows padded as in BlockSmem
  float dl[GM][16];
  float u[GM][16];
  float sx[GM][16];
  float g[GM][16];
  __attribute__((aligned(16))) float b[16][kRow];
  __attribute__((aligned(16))) float c[16][kRow];
  float part[4][GM][16];
  float prod[NQ][16][16];  // [part][state][channel]: product of abar over the part
  float fend[NQ][16][16];  // forward chain from zero, after the part's last token
  float rbeg[NQ][16][16];  // reverse chain from zero, at the part's first token
};

template <typename T, int GM, int NQ>
__global__ __launch_bounds__(256 * NQ) void k_block_parts(const T* __restrict__ x, const T* __restrict__ dt,
                                                          const T* __restrict__ z, const float* __restrict__ A,
                                                          const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                          const float* __restrict__ Dv,
                                                          const float* __restrict__ dt_bias, const float* h_in,
                                                          float* h_out, T* __restrict__ out, int G, int D, int N,
                                                          int flags) {
  constexpr int kThreads = 256 * NQ;
  constexpr int GP = GM / NQ;  // tokens per part
  // every value of a part's tokens stays in registers across the barrier: 16 tokens at most
  static_assert(GP % 4 == 0 && GP <= 16, "parts of 4 to 16 tokens");
  __shared__ BlockSmemParts<GM, NQ> sm;
  const int tid = threadIdx.x;
  const int p = tid / 256;  // part, wavefront-uniform
  const int wv = (tid % 256) / 64;
  const int lane = tid % 64;
  const int cl = lane >> 2;
  const int n = wv * 4 + (lane & 3);
  const int d = blockIdx.x * 16 + cl;
  const int b = blockIdx.y;
  const bool gate = (flags & kNoGate) == 0;
  const bool fwd = (flags & kRevOnly) == 0;
  const bool rev = (flags & kFwdOnly) == 0;

  float av, hv;
  block_stage<T, GM, kThreads>(sm, x, dt, z, A, Bm, Cm, Dv, dt_bias, h_in, G, D, N, gate, fwd && rev, n, d, b, av,
                               hv);
  __syncthreads();

  // phase 1: the part's chains from zero and the running products of abar
  const int t0 = p * GP;
  const float a2 = n < N ? av * kLog2e : 0.0f;
  float a[GP], bb[GP];
#pragma unroll
  for (int t4 = 0; t4 < GP / 4; ++t4) {
    const float4 bq = *reinterpret_cast<const float4*>(&sm.b[n][t0 + 4 * t4]);
    const float bq4[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * t4 + i;
      a[t] = fast_exp2(sm.dl[t0 + t][cl] * a2);
      bb[t] = sm.u[t0 + t][cl] * bq4[i];
    }
  }
  float y[GP], pf[GP], pr[GP];  // y: C_t (hf + hr); pf, pr: C_t times the forward / reverse product
  float hf = 0.0f, qf = 1.0f;
#pragma unroll
  for (int t = 0; t < GP; ++t) {
    hf = fmaf(a[t], hf, bb[t]);
    qf *= a[t];
    y[t] = fwd ? hf : 0.0f;
    pf[t] = qf;
  }
  float hr = 0.0f, qr = 1.0f;
#pragma unroll
  for (int t = GP - 1; t >= 0; --t) {
    hr = fmaf(a[t], hr, bb[t]);
    qr *= a[t];
    if (rev) y[t] += hr;
    pr[t] = qr;
  }
#pragma unroll
  for (int t4 = 0; t4 < GP / 4; ++t4) {
    const float4 cq = *reinterpret_cast<const float4*>(&sm.c[n][t0 + 4 * t4]);
    const float cq4[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * t4 + i;
      y[t] *= cq4[i];
      pf[t] *= cq4[i];
      pr[t] *= cq4[i];
    }
  }
  sm.prod[p][n][cl] = qf;
  sm.fend[p][n][cl] = hf;
  sm.rbeg[p][n][cl] = hr;
  __syncthreads();

  // phase 2: the entering states and each token's corrections
  float hin_f = (n < N && h_in) ? hv : 0.0f;
#pragma unroll
  for (int q = 0; q < NQ - 1; ++q)
    if (q < p) hin_f = fmaf(sm.prod[q][n][cl], hin_f, sm.fend[q][n][cl]);
  float hin_r = 0.0f;
#pragma unroll
  for (int q = NQ - 1; q > 0; --q)
    if (q > p) hin_r = fmaf(sm.prod[q][n][cl], hin_r, sm.rbeg[q][n][cl]);
  if (!fwd) hin_f = 0.0f;
  if (!rev) hin_r = 0.0f;
#pragma unroll
  for (int t = 0; t < GP; ++t) y[t] = quad_sum(fmaf(pf[t], hin_f, fmaf(pr[t], hin_r, y[t])));
  if (p == NQ - 1 && h_out && n < N) {
    // the forward state after the block's last token (padding leaves it unchanged); the entering state is
    // formed again with the cache, whatever the forward readout flag
    float h = h_in ? hv : 0.0f;
#pragma unroll
    for (int q = 0; q < NQ - 1; ++q) h = fmaf(sm.prod[q][n][cl], h, sm.fend[q][n][cl]);
    h_out[(static_cast<size_t>(b) * D + d) * N + n] = fmaf(qf, h, hf);
  }
  if ((lane & 3) == 0) {
#pragma unroll
    for (int t = 0; t < GP; ++t) sm.part[wv][t0 + t][cl] = y[t];
  }
  __syncthreads();
  block_store<T, GM, kThreads>(sm, out, G, D, b);
}

template <typename T, int GM>
static void launch_block_gm(const ScanArgs& a, int batch, int G, int D, int N, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(D / 16), static_cast<unsigned>(batch));
  if constexpr (GM == 32 || GM == 64) {
    // parts of 16 tokens: two (512 threads) or four (1024 threads)
    constexpr int NQ = GM / 16;
    hipLaunchKernelGGL((k_block_parts<T, GM, NQ>), grid, dim3(256 * NQ), 0, stream, static_cast<const T*>(a.x),
                       static_cast<const T*>(a.dt), static_cast<const T*>(a.z), a.A, static_cast<const T*>(a.B),
                       static_cast<const T*>(a.C), a.D, a.dt_bias, a.h_in, a.h_out, static_cast<T*>(a.out), G, D,
                       N, static_cast<int>(a.flags));
  } else {
    constexpr int HV = GM >= 32 ? 2 : 1;  // halves of 16 tokens or more
    hipLaunchKernelGGL((k_block<T, GM, HV>), grid, dim3(256 * HV), 0, stream, static_cast<const T*>(a.x),
                       static_cast<const T*>(a.dt), static_cast<const T*>(a.z), a.A, static_cast<const T*>(a.B),
                       static_cast<const T*>(a.C), a.D, a.dt_bias, a.h_in, a.h_out, static_cast<T*>(a.out), G, D,
                       N, static_cast<int>(a.flags));
  }
}

template <typename T>
static hipError_t launch_block_typed(const ScanArgs& a, int batch, int G, int D, int N, hipStream_t stream) {
  if (G <= 16) {
    launch_block_gm<T, 16>(a, batch, G, D, N, stream);
  } else if (G <= 32) {
    launch_block_gm<T, 32>(a, batch, G, D, N, stream);
  } else if (G <= 64) {
    launch_block_gm<T, 64>(a, batch, G, D, N, stream);
  } else {
    launch_block_gm<T, 128>(a, batch, G, D, N, stream);
  }
  return hipGetLastError();
}

hipError_t launch_block_fused(const ScanArgs& a, int64_t batch, int64_t block_len, int64_t d_inner,
                              int64_t d_state, hipStream_t stream) {
  const int nb = static_cast<int>(batch), G = static_cast<int>(block_len), D = static_cast<int>(d_inner),
            N = static_cast<int>(d_state);
  if (a.io_dtype == 1) return launch_block_typed<bf16_t>(a, nb, G, D, N, stream);
  return launch_block_typed<float>(a, nb, G, D, N, stream);
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <typename T, int NM, int DIRS>
static void launch_output(dim3 grid, hipStream_t stream, const T* x, const T* dt, const T* z, const ScanArgs& a,
                          const float* bct, T* out, int L, int D, int N, int chunk, int nchunk, int nsub, int ntile,
                          int gate, const float* Cf, const float* Cr, const float* R, const float* SIG,
                          const float* A2T) {
  hipLaunchKernelGGL((k_output<T, NM, DIRS>), grid, dim3(64), 0, stream, x, dt, z, a.A, bct, a.D, a.dt_bias, out, L,
                     D, N, chunk, nchunk, nsub, ntile, gate, Cf, Cr, R, SIG, A2T, a.h_out);
}

template <typename T, int NM, int DS>
static void launch_summary(dim3 grid, hipStream_t stream, const T* x, const T* dt, const ScanArgs& a,
                           const float* bct, int L, int D, int N, int chunk, int nchunk, int nsub, int ntile, float* Sf,
                           float* Sr, float* P, float* R, float* SIG) {
  hipLaunchKernelGGL((k_summary<T, NM, DS>), grid, dim3(64), 0, stream, x, dt, a.A, bct, a.dt_bias, L, D, N, chunk,
                     nchunk, nsub, ntile, Sf, Sr, P, R, SIG);
}

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
  float* A2T = reinterpret_cast<float*>(w + p.off_a2t);
  float* bct = reinterpret_cast<float*>(w + p.off_bct);
  const int ntile = static_cast<int>(p.ntile);
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
    const size_t nbc = static_cast<size_t>(p.batch) * ntile * N * kSub;
    hipLaunchKernelGGL((k_stage_bc<T>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, stream, Bm, Cm,
                       bct, L, N, ntile, nbc);
    // the forward summary feeds the forward readout and the cached forward state;
    // the reverse summary feeds the reverse readout
    const bool need_f = (a.flags & kRevOnly) == 0 || a.h_out != nullptr;
    const bool need_r = (a.flags & kFwdOnly) == 0;
    if (need_f && need_r) {
      launch_summary<T, NM, 3>(grid, stream, x, dt, a, bct, L, D, N, chunk, nchunk, nsub, ntile, Sf, Sr, P, R, SIG);
    } else if (need_f) {
      launch_summary<T, NM, 1>(grid, stream, x, dt, a, bct, L, D, N, chunk, nchunk, nsub, ntile, Sf, Sr, P, R, SIG);
    } else {
      launch_summary<T, NM, 2>(grid, stream, x, dt, a, bct, L, D, N, chunk, nchunk, nsub, ntile, Sf, Sr, P, R, SIG);
    }
    e = hipGetLastError();
    if (e != hipSuccess || stage == 0) return e;
  }

  if (stage < 0 || stage == 1) {
    const size_t nthreads = static_cast<size_t>(p.batch) * N * D;
    hipLaunchKernelGGL(k_carry, dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0, stream, Sf, Sr,
                       P, Cf, Cr, a.h_in, a.A, A2T, static_cast<int>(p.batch), nchunk, N, D);
    e = hipGetLastError();
    if (e != hipSuccess || stage == 1) return e;
  }

  const int gate = (a.flags & kNoGate) ? 0 : 1;
  if (a.flags & kFwdOnly) {
    launch_output<T, NM, 1>(grid, stream, x, dt, z, a, bct, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf,
                            Cr, R, SIG, A2T);
  } else if ((a.flags & kRevOnly) && a.h_out != nullptr) {
    // the cached forward state needs the forward chain: left to right, reverse from the boundary states
    launch_output<T, NM, 2>(grid, stream, x, dt, z, a, bct, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf,
                            Cr, R, SIG, A2T);
  } else if (a.flags & kRevOnly) {
    launch_output<T, NM, 6>(grid, stream, x, dt, z, a, bct, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf,
                            Cr, R, SIG, A2T);
  } else {
    launch_output<T, NM, 3>(grid, stream, x, dt, z, a, bct, out, L, D, N, chunk, nchunk, nsub, ntile, gate, Cf,
                            Cr, R, SIG, A2T);
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
