// Short causal / anti-causal depthwise convolution with SiLU, both directions
// from one read of the input, for gfx950.
//
// Operation: the Conv1d of width d_conv = 4 that each direction of the
// DiffuMamba mixer runs ahead of its scan ("DiffuMamba: High-Throughput
// Diffusion LMs with Mamba Backbone", arXiv v4, Appendix C Table 12; width and
// untied directions in Section 4.1 Table 8; the reverse layer is the forward
// one on the flipped sequence, Section 3.2):
//   fwd[t, c] = silu(b_f[c] + sum_k w_f[c, k] * u[t - 3 + k, c])
//   rev[t, c] = silu(b_r[c] + sum_k w_r[c, k] * u[t + 3 - k, c])
// with u = 0 outside the sequence, or in block decoding u before the block
// taken from a 3-token cache and u after the block taken as 0 (Section 4.3,
// block-cache paragraph).
//
// One thread owns 4 channels of a 64-token tile.  It walks the tile in blocks
// of 8 tokens with a 14-row window in registers (the 3 rows before the block,
// the block, and 3 rows after it), loading the rows of the next block while it
// computes the current one, so every input row is read once (plus a 6-row halo
// per tile) and both outputs are written once: the kernel is a pure HBM stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "launch.h"

namespace bimamba {
namespace conv {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // tokens per thread
constexpr int kBlk = 8;     // tokens per window step
constexpr int kK = 4;       // filter width
constexpr int kWin = kBlk + 2 * (kK - 1);

// 4 consecutive elements of one row, as fp32.
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x;
  v[1] = q.y;
  v[2] = q.z;
  v[3] = q.w;
}

__device__ __forceinline__ void load4(const bf16_t* p, float v[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// round to nearest even, two values per v_cvt_pk_bf16_f32
__device__ __forceinline__ void store4(bf16_t* p, const float v[4]) {
  const f32x4 f = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, __builtin_convertvector(f, bf16x4));
}

// Buffer resources.  A tile's first row is the base of its resources and the
// row offset goes into the VGPR offset together with the lane's channels.  The
// hardware range check of a raw buffer access (offset >= num_records: a load
// returns 0, a store is dropped) supplies the zero padding past the sequence end
// and drops the outputs past it, so no access needs a guard.
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor, untyped 32-bit data format
// u and both outputs are streamed through once: non-temporal (the nt bit of the cache-policy field)
constexpr int kStream = 2;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kRsrcWord3);
}

// Raw 4-element row chunks, kept undecoded while a load is in flight.
template <typename T>
struct Raw;

template <>
struct Raw<float> {
  u32x4 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream);
  }
  __device__ __forceinline__ void get(float o[4]) const {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
  using Word = u32x4;
  static __device__ __forceinline__ Word pack(const float o[4]) {
    return Word{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
  }
  static __device__ __forceinline__ void store_word(Word q, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, kStream);
  }
  static __device__ __forceinline__ void store(const float o[4], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    store_word(pack(o), r, off);
  }
};

template <>
struct Raw<bf16_t> {
  u32x2 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStream);
  }
  __device__ __forceinline__ void get(float o[4]) const {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  // round to nearest even, two values per v_cvt_pk_bf16_f32
  using Word = u32x2;
  static __device__ __forceinline__ Word pack(const float o[4]) {
    const f32x4 f = {o[0], o[1], o[2], o[3]};
    return __builtin_bit_cast(u32x2, __builtin_convertvector(f, bf16x4));
  }
  static __device__ __forceinline__ void store_word(Word q, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(q, r, off, 0, kStream);
  }
  static __device__ __forceinline__ void store(const float o[4], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    store_word(pack(o), r, off);
  }
};

__device__ __forceinline__ void copy4(float* dst, const float* src) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = src[i];
}

template <typename T>
struct Args {
  const T* u;          // [batch, L, C]
  const float* w_f;    // [C, 4]
  const float* b_f;    // [C] or null
  const float* w_r;
  const float* b_r;
  const T* cache_in;   // [batch, 3, C] or null (block decoding)
  T* cache_out;        // [batch, 3, C] or null
  T* out_f;            // [batch, L, C] or null
  T* out_r;
  int64_t L, C;
};

template <bool ACT>
__device__ __forceinline__ float act_f32(float s) {
  return ACT ? silu_f32(s) : s;
}

template <typename T, bool ACT>
__global__ __launch_bounds__(kThreads) void k_conv(Args<T> a) {
  // workgroups walk the channel blocks of a tile first, so that the ones in flight read whole rows
  const int64_t cblocks = (a.C / 4 + kThreads - 1) / kThreads;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) / cblocks;
  const int64_t c0 = ((static_cast<int64_t>(blockIdx.x) - tile * cblocks) * kThreads + threadIdx.x) * 4;
  if (c0 >= a.C) return;  // no barriers below
  const int64_t t0 = tile * kTile;
  const int64_t b = blockIdx.y;
  const bool do_f = a.out_f != nullptr, do_r = a.out_r != nullptr;

  float wf[4][kK], wr[4][kK], bfv[4], brv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int k = 0; k < kK; ++k) {
      wf[i][k] = do_f ? a.w_f[(c0 + i) * kK + k] : 0.0f;
      wr[i][k] = do_r ? a.w_r[(c0 + i) * kK + k] : 0.0f;
    }
    bfv[i] = (do_f && a.b_f) ? a.b_f[c0 + i] : 0.0f;
    brv[i] = (do_r && a.b_r) ? a.b_r[c0 + i] : 0.0f;
  }

  // row t of the (cache ++ sequence ++ zeros) input, channels c0..c0+3 (tile edges only)
  auto row = [&](int64_t t, float v[4]) {
    if (t >= 0 && t < a.L) {
      load4(a.u + (b * a.L + t) * a.C + c0, v);
    } else if (t < 0 && t >= -(kK - 1) && a.cache_in) {
      load4(a.cache_in + (b * (kK - 1) + (kK - 1) + t) * a.C + c0, v);
    } else {
      v[0] = v[1] = v[2] = v[3] = 0.0f;
    }
  };

  // this tile's rows t0 .. t0 + 66 (its tokens and the 3 after them) and its output rows t0 .. t0 + 63;
  // the resources end at the sequence end
  const uint32_t row_bytes = static_cast<uint32_t>(a.C) * static_cast<uint32_t>(sizeof(T));
  const int64_t left = a.L - t0;
  const uint32_t in_rows = static_cast<uint32_t>(left < kTile + kK - 1 ? left : kTile + kK - 1);
  const uint32_t out_rows = static_cast<uint32_t>(left < kTile ? left : kTile);
  const int64_t base = (b * a.L + t0) * a.C;
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.u + base, in_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rf = make_rsrc(do_f ? a.out_f + base : nullptr, do_f ? out_rows * row_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(do_r ? a.out_r + base : nullptr, do_r ? out_rows * row_bytes : 0u);
  const uint32_t lane_off = static_cast<uint32_t>(c0) * static_cast<uint32_t>(sizeof(T));

  float win[kWin][4];  // win[m] = row t_blk - 3 + m
#pragma unroll
  for (int m = 0; m < kK - 1; ++m) row(t0 - (kK - 1) + m, win[m]);
  {
    Raw<T> q[kK - 1];
#pragma unroll
    for (int m = 0; m < kK - 1; ++m) q[m].load(ru, lane_off + m * row_bytes);
#pragma unroll
    for (int m = 0; m < kK - 1; ++m) q[m].get(win[kK - 1 + m]);
  }
  // the rows a block adds to the window are loaded one block ahead
  Raw<T> nxt[kBlk];
  auto fetch = [&](int blk) {
#pragma unroll
    for (int m = 0; m < kBlk; ++m) nxt[m].load(ru, lane_off + (blk * kBlk + (kK - 1) + m) * row_bytes);
  };
  fetch(0);
  // bf16: a block's outputs are stored during the next block, right after its rows are fetched, so
  // that the wait for those rows (vector memory completes in order) never waits for the stores
  constexpr bool kDefer = sizeof(T) == 2;
  typename Raw<T>::Word pf[kDefer ? kBlk : 1], pr[kDefer ? kBlk : 1];
  auto flush = [&](int blk) {
#pragma unroll
    for (int tt = 0; tt < kBlk; ++tt) {
      const uint32_t off = lane_off + (blk * kBlk + tt) * row_bytes;
      if (do_f) Raw<T>::store_word(pf[kDefer ? tt : 0], rf, off);
      if (do_r) Raw<T>::store_word(pr[kDefer ? tt : 0], rr, off);
    }
  };
  int nblk = 0;  // blocks computed
  for (int blk = 0; blk < kTile / kBlk; ++blk) {
    if (t0 + blk * kBlk >= a.L) break;
#pragma unroll
    for (int m = 0; m < kBlk; ++m) nxt[m].get(win[2 * (kK - 1) + m]);
    if (blk + 1 < kTile / kBlk) fetch(blk + 1);
    if (kDefer && blk > 0) flush(blk - 1);
#pragma unroll
    for (int tt = 0; tt < kBlk; ++tt) {
      const uint32_t off = lane_off + (blk * kBlk + tt) * row_bytes;
      if (do_f) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = bfv[i];
#pragma unroll
          for (int k = 0; k < kK; ++k) s = fmaf(wf[i][k], win[tt + k][i], s);
          o[i] = act_f32<ACT>(s);
        }
        if (kDefer) pf[kDefer ? tt : 0] = Raw<T>::pack(o);
        else Raw<T>::store(o, rf, off);
      }
      if (do_r) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = brv[i];
#pragma unroll
          for (int k = 0; k < kK; ++k) s = fmaf(wr[i][k], win[tt + 2 * (kK - 1) - k][i], s);
          o[i] = act_f32<ACT>(s);
        }
        if (kDefer) pr[kDefer ? tt : 0] = Raw<T>::pack(o);
        else Raw<T>::store(o, rr, off);
      }
    }
#pragma unroll
    for (int m = 0; m < 2 * (kK - 1); ++m) copy4(win[m], win[kBlk + m]);
    ++nblk;
  }
  if (kDefer && nblk > 0) flush(nblk - 1);

  // The cache for the next block: the last 3 rows of (cache ++ sequence).  Only this thread touches
  // these channels of the caches, and it reads all three rows before it writes any, so cache_out
  // may alias cache_in.
  if (tile == 0 && a.cache_out) {
    float v[kK - 1][4];
#pragma unroll
    for (int m = 0; m < kK - 1; ++m) row(a.L - (kK - 1) + m, v[m]);
#pragma unroll
    for (int m = 0; m < kK - 1; ++m) store4(a.cache_out + (b * (kK - 1) + m) * a.C + c0, v[m]);
  }
}

template <typename T, bool ACT>
hipError_t launch_t(const ConvArgs& in, int64_t batch, int64_t L, int64_t C, hipStream_t stream) {
  Args<T> a{};
  a.u = static_cast<const T*>(in.u);
  a.w_f = in.w_f;
  a.b_f = in.b_f;
  a.w_r = in.w_r;
  a.b_r = in.b_r;
  a.cache_in = static_cast<const T*>(in.cache_in);
  a.cache_out = static_cast<T*>(in.cache_out);
  a.out_f = static_cast<T*>(in.out_f);
  a.out_r = static_cast<T*>(in.out_r);
  a.L = L;
  a.C = C;
  const int64_t cblocks = (C / 4 + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<unsigned>((L + kTile - 1) / kTile * cblocks), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((k_conv<T, ACT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_act(const ConvArgs& in, int64_t batch, int64_t L, int64_t C, hipStream_t stream) {
  return in.act ? launch_t<T, true>(in, batch, L, C, stream) : launch_t<T, false>(in, batch, L, C, stream);
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, int64_t batch, int64_t L, int64_t C, int io_dtype, hipStream_t stream) {
  return io_dtype == 1 ? launch_act<bf16_t>(a, batch, L, C, stream) : launch_act<float>(a, batch, L, C, stream);
}

}  // namespace conv
}  // namespace bimamba
