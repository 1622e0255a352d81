// Bidirectional Mamba-2 (SSD) scan for gfx950 on the matrix cores.
//
// Operation: "DiffuMamba: High-Throughput Diffusion LMs with Mamba Backbone"
// (arXiv v4), Section 3.2 eq. (4)-(6) with the Mamba-2 mixer of Section 1:
// heads of 32 channels, a scalar transition abar = exp(delta * A[h]) per
// (token, head), delta = softplus(dt + dt_bias[h]), B_t and C_t (state size
// 128) shared by all heads, readout C . state + D[h] x per direction, the two
// directions summed and gated by SiLU(z) (Appendix A Table 7; Appendix C
// Table 12 and its caption).
//
// Because the transition is a scalar per head, a run of Q = 64 tokens is a
// handful of dense products (s = running sum of delta*A inside the run, e the
// exclusive one, S the run total, "o" = outer product over (channel, state)):
//   intra-run   y_i += sum_j  W_ij (C_i . B_j) delta_j x_j, with
//                 W_ij = exp(s_i - s_j) for j < i (forward), exp(e_j - e_i)
//                 for j > i (reverse), and the number of directions on the
//                 diagonal;
//   readout     y_i += exp(s_i) C_i . H_in      (forward state entering the run)
//               y_i += exp(S - e_i) C_i . G_in  (reverse state entering from the right)
//   update      H_out = exp(S) H_in + sum_j exp(S - s_j) delta_j x_j o B_j
//               G_out = exp(S) G_in + sum_j exp(e_j) delta_j x_j o B_j
// The products take bf16 operands with fp32 accumulation
// (v_mfma_f32_16x16x32_bf16); the states stay in fp32 accumulators and only
// their operand copies are rounded to bf16.
//
// Passes (the sequence is cut into chunks of whole runs):
//   k_ssd_stage   per run: C into a zero-padded tile, B transposed (the state
//                 update contracts over tokens), and C B^T in fp32 (it does not
//                 depend on the head, so it is formed once here).
//   k_ssd_rsweep  per (chunk, head), right to left over the runs: the
//                 intra-run products of both directions plus the readout of
//                 the reverse state from zero at the chunk end; this partial
//                 output goes to `out` in bf16.  It also leaves the chunk's
//                 forward end state and reverse start state from zero, the
//                 product of abar over the chunk, and for every run the product
//                 of abar over the chunk's tokens to its right.
//   k_ssd_carry   chains the chunk maps across the sequence in both directions.
//   k_ssd_fsweep  per (chunk, head), left to right: adds the readout of the
//                 forward state, the readout of the reverse state entering the
//                 chunk from the right (decayed to each token), the skip term
//                 and the gate, and writes `out`.
// Both sweeps keep the next run's global data in flight while the current run
// computes: a step commits the registers loaded during the previous step to
// LDS, issues the next step's loads, then computes; one wavefront forms the
// next run's per-token terms at the end of the step.  Two workgroups fit on a
// CU, so one computes while the other waits.
//
// Also here: the block-cache step in one kernel (k_ssd_block), and the
// one-direction layers with the short convolution applied on load (k_ssd1_*),
// each described at its definition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"
#include "launch.h"
#include "ssd_plan.h"

namespace bimamba {
namespace ssd {

namespace {

constexpr int P = static_cast<int>(kHeadDim);
constexpr int N = static_cast<int>(kState);
constexpr int Q = static_cast<int>(kQ);
constexpr int kSF = static_cast<int>(kStateFloats);
constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes (arrays of it stay in registers)

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

__device__ __forceinline__ uint16_t to_bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16 bytes of a run's output (token 16w + l/4 of the run, channels 8(l%4)..+7 of head h) through a
// buffer resource whose range ends at the sequence end: rows past it are dropped by the hardware, so
// the store is issued by every lane without a branch.
__device__ __forceinline__ void store_run_row(uint16_t* out, int64_t b, int64_t L, int64_t HP, int64_t t0,
                                              int64_t h, int row, int part, uint4 v) {
  const int64_t nv = L - t0 < Q ? L - t0 : Q;  // valid tokens of the run
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(out + (b * L + t0) * HP + h * P, static_cast<short>(0),
                                                               static_cast<int>(nv * HP * 2), 0x00020000);
  const uint32_t off = static_cast<uint32_t>((row * HP + 8 * part) * 2);
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}

// LDS tiles of bf16 rows, in 16-byte chunks of 8 elements.  Chunk c of row r is
// stored at a swizzled chunk position so that 16 lanes reading the same chunk
// of 16 consecutive rows hit different banks.
__device__ __forceinline__ int sw256(int r, int c) { return r * 128 + ((c ^ (r & 15)) << 3); }      // 128-element rows
__device__ __forceinline__ int sw128(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }  // 64-element rows

__device__ __forceinline__ bf16x8 lds8(const uint16_t* s, int idx) {
  return *reinterpret_cast<const bf16x8*>(s + idx);
}

__device__ __forceinline__ float ex(float v) { return fast_exp2(v * kLog2e); }

// s_waitcnt vmcnt(0): every vector memory operation this wavefront issued is complete (direct-to-LDS loads
// included, which the compiler does not track); the empty asm keeps LDS accesses from moving across it.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt at their maxima (not waited for)
  asm volatile("" ::: "memory");
}

// Per-token quantities of one run, one lane per token, in LDS rows of 64.
enum Tok { kDl = 0, kS, kE, kWr, kWf, kRr, kRf, kTokRows };

struct Args {
  const uint16_t* x;   // [batch, L, H*P]
  const uint16_t* dt;  // [batch, L, H]
  const float* A;      // [H]
  const uint16_t* B;   // [batch, L, N]
  const uint16_t* C;
  const float* D;      // [H] or null
  const uint16_t* z;   // [batch, L, H*P] or null
  const float* dt_bias;
  uint16_t* out;       // [batch, L, H*P]; holds the reverse sweep's partial output between the sweeps
  int64_t L, H;
  int64_t nsub, rpc, nchunk;
  float* g;       // [batch, nsub, 4, 4, 64, 4]: C B^T per run in accumulator order
  uint16_t* cp;   // [batch, nsub, Q, N]
  uint16_t* bt;   // [batch, nsub, N, Q]
  float* S;       // [batch, nchunk, H, 2, kSF]  (chunk-local, then entering states)
  float* Pc;      // [batch, nchunk, H]
  float* tau;     // [batch, nchunk, H, rpc]: product of abar over the chunk's tokens right of each run
  int gate;
  const float* h_in;  // [batch, H, P, N] forward state entering the sequence, or null (zeros)
  float* h_out;       // [batch, H, P, N] forward state after the sequence, or null
  // one-direction layers only: x (and B, C) are columns of one projection stream of xs elements per token
  // (x = channels [0, H*P), B = [H*P, H*P+N), C = [H*P+N, H*P+2N)); cw [xs, 4] and cb [xs] are the short
  // convolution's taps and bias (cw null: no convolution, cb null: no bias)
  int64_t xs;
  const float* cw;
  const float* cb;
};

// (batch, chunk, head) of a workgroup.  Workgroups are dispatched round-robin
// over the 8 XCDs; the mapping gives each XCD a contiguous range of
// (chunk, head) items, chunk-major, so the heads of a chunk share one L2 for
// the chunk's tiles.
__device__ __forceinline__ void decode_item(const Args& a, int64_t& b, int64_t& c, int64_t& h) {
  const int64_t total = static_cast<int64_t>(gridDim.x);
  const int64_t i = blockIdx.x;
  const int64_t item = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
  h = item % a.H;
  c = (item / a.H) % a.nchunk;
  b = item / (a.H * a.nchunk);
}

__device__ __forceinline__ uint16_t load_dt(const Args& a, int64_t b, int64_t t0, int64_t h, int l) {
  return (t0 + l < a.L) ? a.dt[(b * a.L + t0 + l) * a.H + h] : static_cast<uint16_t>(0);
}

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts within rows of 16 lanes (DPP row_shr, lanes
// shifted in from outside the row read 0), then each row's total carried into the rows after it (DPP
// row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3; rows left out of the row mask add 0).
template <int CTRL, int ROW_MASK, bool BOUND0>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, BOUND0));
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_f32<0x111, 0xf, true>(v);   // row_shr:1
  v += dpp_f32<0x112, 0xf, true>(v);   // row_shr:2
  v += dpp_f32<0x114, 0xf, true>(v);   // row_shr:4
  v += dpp_f32<0x118, 0xf, true>(v);   // row_shr:8
  v += dpp_f32<0x142, 0xa, false>(v);  // row_bcast:15
  v += dpp_f32<0x143, 0xc, false>(v);  // row_bcast:31
  return v;
}

// One run's per-token quantities, computed by one wavefront (lane = token).
// Tokens past the sequence end get delta = 0: no decay and no input.
__device__ __forceinline__ void token_prep(float* tok, uint16_t dtv, bool valid, float Ah, float bias, int l) {
  const float dl = valid ? softplus_f32(bf(dtv) + bias) : 0.0f;
  const float av = dl * Ah;
  const float s = wave_prefix_sum(av);
  const float S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
  const float e = s - av;
  tok[kDl * 64 + l] = dl;
  tok[kS * 64 + l] = s;
  tok[kE * 64 + l] = e;
  tok[kWr * 64 + l] = ex(e) * dl;
  tok[kWf * 64 + l] = ex(S - s) * dl;
  tok[kRr * 64 + l] = ex(S - e);
  tok[kRf * 64 + l] = ex(s);
}

// The decay mask on wavefront w's block tj of C B^T (rows i = 16w + l16, columns j = j0 + r, j0 = 16tj + 4q4),
// times delta_j: forward e^{s_i - s_j} below the diagonal, reverse e^{e_j - e_i} above it, `diag` on it.  A
// block lies wholly below the diagonal when tj < w and wholly above it when tj > w; w is wavefront-uniform, so
// only the diagonal block selects per lane.
template <bool FWD, bool REV>
__device__ __forceinline__ void mask_block(f32x4& g, int tj, int w, int i, int j0, float si, float ei,
                                           const f32x4& sj, const f32x4& ej, const f32x4& dj, float diag) {
  if (tj < w) {
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = FWD ? g[r] * (ex(si - sj[r]) * dj[r]) : 0.0f;
  } else if (tj > w) {
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r] = REV ? g[r] * (ex(ej[r] - ei) * dj[r]) : 0.0f;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + r;
      float m;
      if (j < i) m = FWD ? ex(si - sj[r]) : 0.0f;
      else if (j > i) m = REV ? ex(ej[r] - ei) : 0.0f;
      else m = diag;
      g[r] *= m * dj[r];
    }
  }
}

// 16 bytes of a [batch, L, H*P] tensor: token t0 + j of the run with j = q/4 and
// channels 8(q%4)..+7 of head h; zero past the sequence end.
__device__ __forceinline__ uint4 load_act(const uint16_t* base, const Args& a, int64_t b, int64_t t0, int64_t h,
                                          int q) {
  const int j = q >> 2, pc = q & 3;
  if (t0 + j >= a.L) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(base + (b * a.L + t0 + j) * (a.H * P) + h * P + 8 * pc);
}

// Thread tid's x chunk (token j = tid/4, channels 8(tid%4)..+7) into LDS rows of
// 64 tokens per channel; scaled by a per-token weight when wtok is given.
__device__ __forceinline__ void put_xt(uint16_t* dst, uint4 v, int tid, const float* wtok, float wscale) {
  const int j = tid >> 2, pc = tid & 3;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const float f = wtok ? wtok[j] * wscale : 1.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t raw = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
    dst[sw128(8 * pc + e, j >> 3) + (j & 7)] = wtok ? to_bf(bf(raw) * f) : raw;
  }
}

// An fp32 value as a pair of bf16 operands, hi = bf16(v) and lo = bf16(v - hi) (both rounded to nearest
// even): hi + lo carries v to about 2^-17 relative, so a product taken as hi * b + lo * b on the matrix cores
// loses no more than that to its operand's rounding (b exact in bf16).
__device__ __forceinline__ uint16_t bf_rest(float v, uint16_t hi) { return to_bf(v - bf(hi)); }

// put_xt's weighted copy as two tiles, the rounded values and their rounding residuals.
__device__ __forceinline__ void put_xt_split(uint16_t* dst, uint16_t* dst_lo, uint4 v, int tid, const float* wtok) {
  const int j = tid >> 2, pc = tid & 3;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const float f = wtok[j];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = bf(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)))) * f;
    const uint16_t hi = to_bf(x);
    const int o = sw128(8 * pc + e, j >> 3) + (j & 7);
    dst[o] = hi;
    dst_lo[o] = bf_rest(x, hi);
  }
}

// Head states are held transposed (rows = state index n, columns = channel p)
// in 16x16 accumulator tiles.  Tile (nb, tp) element r in lane l is
// n = 16nb + 4(l/16) + r, p = 16tp + l%16; in memory a state is stored as
// [nb][tp][lane][r] (nb = 0..7, tp = 0..1), 4096 floats.  Wavefront w of a
// workgroup owns the row blocks nb = 2w and 2w + 1.
__device__ __forceinline__ int state_off(int nb, int tp, int l) { return ((nb * 2 + tp) * 64 + l) * 4; }

struct State {
  f32x4 t[2][2];  // [row block 2w + i][channel tile]
};

__device__ __forceinline__ void state_load(State& s, const float* g, int w, int l) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) s.t[i][tp] = *reinterpret_cast<const f32x4*>(g + state_off(2 * w + i, tp, l));
}

__device__ __forceinline__ void state_store(const State& s, float* g, int w, int l) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) *reinterpret_cast<f32x4*>(g + state_off(2 * w + i, tp, l)) = s.t[i][tp];
}

__device__ __forceinline__ void state_zero(State& s) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) s.t[i][tp] = zero4();
}

// bf16 copy of the wavefront's part of a state into LDS rows p of 128 states
// (the B operand of the readout).
__device__ __forceinline__ void state_to_lds(const State& s, uint16_t* sHs, int w, int l) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const f32x4 v = s.t[i][tp];
      const int p = 16 * tp + (l & 15);
      const int n0 = 16 * (2 * w + i) + 4 * (l >> 4);
      const uint32_t lo = static_cast<uint32_t>(to_bf(v[0])) | (static_cast<uint32_t>(to_bf(v[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(to_bf(v[2])) | (static_cast<uint32_t>(to_bf(v[3])) << 16);
      *reinterpret_cast<uint2*>(sHs + sw256(p, n0 >> 3) + (n0 & 7)) = make_uint2(lo, hi);
    }
}

// state_to_lds as two copies, the rounded state (sHs) and its rounding residuals (sHr).
__device__ __forceinline__ void state_to_lds_split(const State& s, uint16_t* sHs, uint16_t* sHr, int w, int l) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const f32x4 v = s.t[i][tp];
      const int p = 16 * tp + (l & 15);
      const int n0 = 16 * (2 * w + i) + 4 * (l >> 4);
      uint16_t hb[4], rb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hb[r] = to_bf(v[r]);
        rb[r] = bf_rest(v[r], hb[r]);
      }
      const int o = sw256(p, n0 >> 3) + (n0 & 7);
      *reinterpret_cast<uint2*>(sHs + o) = make_uint2(hb[0] | (static_cast<uint32_t>(hb[1]) << 16),
                                                      hb[2] | (static_cast<uint32_t>(hb[3]) << 16));
      *reinterpret_cast<uint2*>(sHr + o) = make_uint2(rb[0] | (static_cast<uint32_t>(rb[1]) << 16),
                                                      rb[2] | (static_cast<uint32_t>(rb[3]) << 16));
    }
}

// state = scale * state + B^T (weighted x): contraction over the run's 64 tokens.
__device__ __forceinline__ void state_update(State& s, float scale, const uint16_t* sBT, const uint16_t* sXW, int w,
                                             int l) {
  const int q4 = l >> 4, l16 = l & 15;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) s.t[i][tp] *= scale;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    bf16x8 xb[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) xb[tp] = lds8(sXW, sw128(16 * tp + l16, 4 * k + q4));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16x8 ab = lds8(sBT, sw128(16 * (2 * w + i) + l16, 4 * k + q4));
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) s.t[i][tp] = mfma(ab, xb[tp], s.t[i][tp]);
    }
  }
}

// y tiles of the wavefront (rows i = 16w + 4(l/16) + r, channels p = 16tp + l%16)
// = C_i . state(p, :), with cf the wavefront's C rows as A operands.
__device__ __forceinline__ void readout(f32x4 y[2], const bf16x8 cf[4], const uint16_t* sHs, int l) {
  const int q4 = l >> 4, l16 = l & 15;
  y[0] = y[1] = zero4();
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) y[tp] = mfma(cf[k], lds8(sHs, sw256(16 * tp + l16, 4 * k + q4)), y[tp]);
}

// The wavefront's 16 x 32 output tile goes through its LDS slot (rows of 32
// bf16) so that each lane moves 16 contiguous bytes.
__device__ __forceinline__ void tile_rows_to_lds(uint16_t* slot, const float v[2][4], int l) {
  const int q4 = l >> 4, l16 = l & 15;
#pragma unroll
  for (int tp = 0; tp < 2; ++tp)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bf16_t ob;
      from_f32(v[tp][r], &ob);
      slot[(4 * q4 + r) * P + 16 * tp + l16] = ob.bits;
    }
}

// The wavefront's C rows i = 16w + l%16 as readout A operands, straight from the
// run's zero-padded C tile: operand kk holds states 32kk + 8(l/16) .. +7.
__device__ __forceinline__ void load_cfrag(u32x4 cf[4], const uint16_t* ctile, int w, int l) {
  const uint16_t* row = ctile + (16 * w + (l & 15)) * N + 8 * (l >> 4);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) cf[kk] = *reinterpret_cast<const u32x4*>(row + 32 * kk);
}

// ---------------------------------------------------------------------------
// k_ssd_stage: per run, C -> zero-padded tile [Q][N], B -> B^T [N][Q], and
// G = C B^T in fp32, stored per 16-row block of i in accumulator order:
// g[ib][tj][lane][r] = C_i . B_j with i = 16ib + lane%16, j = 16tj + 4(lane/16) + r.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_ssd_stage(const uint16_t* Bm, const uint16_t* Cm, float* g,
                                                        uint16_t* cp, uint16_t* bt, int64_t L, int64_t nsub) {
  __shared__ __attribute__((aligned(16))) uint16_t sBs[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sCs[Q * N];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  const int64_t sub = blockIdx.x, b = blockIdx.y;
  const int64_t t0 = sub * Q;
  const int64_t tile = (b * nsub + sub) * static_cast<int64_t>(Q * N);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int j = ci >> 4, cc = ci & 15;
    uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
    if (t0 + j < L) {
      vb = *reinterpret_cast<const uint4*>(Bm + (b * L + t0 + j) * N + 8 * cc);
      vc = *reinterpret_cast<const uint4*>(Cm + (b * L + t0 + j) * N + 8 * cc);
    }
    *reinterpret_cast<uint4*>(cp + tile + j * N + 8 * cc) = vc;
    *reinterpret_cast<uint4*>(sBs + sw256(j, cc)) = vb;
    *reinterpret_cast<uint4*>(sCs + sw256(j, cc)) = vc;
  }
  __syncthreads();
  // B^T rows n, 8 tokens per 16-byte chunk
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int n = ci >> 3, jc = ci & 7;
    uint32_t w2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = 8 * jc + 2 * e;
      w2[e] = static_cast<uint32_t>(sBs[sw256(j0, n >> 3) + (n & 7)]) |
              (static_cast<uint32_t>(sBs[sw256(j0 + 1, n >> 3) + (n & 7)]) << 16);
    }
    *reinterpret_cast<uint4*>(bt + tile + n * Q + 8 * jc) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
  }
  // C B^T: wavefront w forms the 4 tiles of row block ib = w
  bf16x8 cf[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cf[k] = lds8(sCs, sw256(16 * w + l16, 4 * k + q4));
  float* gout = g + (b * nsub + sub) * static_cast<int64_t>(Q * Q);
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    f32x4 acc = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = mfma(lds8(sBs, sw256(16 * tj + l16, 4 * k + q4)), cf[k], acc);
    *reinterpret_cast<f32x4*>(gout + ((w * 4 + tj) * 64 + l) * 4) = acc;
  }
}

// ---------------------------------------------------------------------------
// k_ssd_rsweep: right to left over a chunk's runs.  Wavefront w owns output
// rows i in [16w, 16w+16) (both channel tiles) and state row blocks 2w, 2w+1.
// DIRS bit 0 = forward, bit 1 = reverse.
// ---------------------------------------------------------------------------
template <int DIRS>
__global__ __launch_bounds__(kThreads, 2) void k_ssd_rsweep(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXWr[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXWf[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sHs[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sOut[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) float sTok[2][kTokRows * 64];
  constexpr bool kFwd = DIRS & 1, kRev = DIRS & 2;
  constexpr float kDiag = (kFwd && kRev) ? 2.0f : 1.0f;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  int64_t b, c, h;
  decode_item(a, b, c, h);
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const int64_t sub0 = c * a.rpc;
  const int64_t nrun = a.nsub - sub0 < a.rpc ? a.nsub - sub0 : a.rpc;
  const int64_t item = (b * a.nchunk + c) * a.H + h;
  uint16_t* slot = sOut + w * 16 * P;
  State G, F;
  state_zero(G);
  state_zero(F);
  float tau = 1.0f;  // product of abar over the chunk's tokens to the right of the current run

  // step st handles run k = nrun-1-st; its loads are issued one step ahead
  u32x4 pc[4], pbt[4];
  f32x4 pg[4];
  uint4 px;
  // step sizes run two steps ahead of the other loads, so that forming the next run's per-token terms
  // at the end of a step never waits for the loads issued in that step
  uint16_t pdt = 0, pdt2 = 0;
  auto issue = [&](int64_t st) {
    const int64_t sub = sub0 + (nrun - 1 - st);
    if (w == 0 && st + 1 < nrun) pdt2 = load_dt(a, b, (sub - 1) * Q, h, l);
    const int64_t tile = (b * a.nsub + sub) * static_cast<int64_t>(Q * N);
    const u32x4* b4 = reinterpret_cast<const u32x4*>(a.bt + tile);
    if (kRev) load_cfrag(pc, a.cp + tile, w, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) pbt[i] = b4[tid + kThreads * i];
    const float* gg = a.g + (b * a.nsub + sub) * static_cast<int64_t>(Q * Q);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) pg[tj] = *reinterpret_cast<const f32x4*>(gg + ((w * 4 + tj) * 64 + l) * 4);
    px = load_act(a.x, a, b, sub * Q, h, tid);
  };
  if (w == 0) pdt = load_dt(a, b, (sub0 + nrun - 1) * Q, h, l);
  issue(0);
  if (w == 0) token_prep(sTok[0], pdt, (sub0 + nrun - 1) * Q + l < a.L, Ah, bias, l);
  pdt = pdt2;

  for (int64_t st = 0; st < nrun; ++st) {
    const int64_t k = nrun - 1 - st;
    const int64_t t0 = (sub0 + k) * Q;
    const float* tok = sTok[st & 1];
    f32x4 gcur[4];
    bf16x8 cf[4];
    __syncthreads();
    // ---- commit the prefetched registers ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(sBT + sw128(ci >> 3, ci & 7)) = pbt[i];
      if (kRev) cf[i] = __builtin_bit_cast(bf16x8, pc[i]);
    }
    put_xt(sXT, px, tid, nullptr, 1.0f);
    if (kRev) put_xt(sXWr, px, tid, tok + kWr * 64, 1.0f);
    if (kFwd) put_xt(sXWf, px, tid, tok + kWf * 64, tau);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) gcur[tj] = pg[tj];
    if (kRev) state_to_lds(G, sHs, w, l);
    __syncthreads();
    if (st + 1 < nrun) issue(st + 1);

    // ---- compute ----
    // W = mask o (C B^T) o delta_j for rows i = 16w + l16, used as the A operand with permuted
    // k-slots: slot e < 4 -> j = 32k2 + 4q4 + e, slot e >= 4 -> j = 32k2 + 16 + 4q4 + e - 4
    const int i = 16 * w + l16;
    const float si = tok[kS * 64 + i], ei = tok[kE * 64 + i];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int j0 = 16 * tj + 4 * q4;
      const f32x4 sj = *reinterpret_cast<const f32x4*>(tok + kS * 64 + j0);
      const f32x4 ej = *reinterpret_cast<const f32x4*>(tok + kE * 64 + j0);
      const f32x4 dj = *reinterpret_cast<const f32x4*>(tok + kDl * 64 + j0);
      mask_block<kFwd, kRev>(gcur[tj], tj, __builtin_amdgcn_readfirstlane(w), i, j0, si, ei, sj, ej, dj, kDiag);
    }
    f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 wa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wa[r] = static_cast<__bf16>(gcur[2 * k2][r]);
        wa[4 + r] = static_cast<__bf16>(gcur[2 * k2 + 1][r]);
      }
      const int jlo = 32 * k2 + 4 * q4;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int p = 16 * tp + l16;
        const uint2 lo = *reinterpret_cast<const uint2*>(sXT + sw128(p, jlo >> 3) + (jlo & 7));
        const uint2 hi = *reinterpret_cast<const uint2*>(sXT + sw128(p, (jlo + 16) >> 3) + (jlo & 7));
        y[tp] = mfma(wa, __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), y[tp]);
      }
    }
    if (kRev) {
      f32x4 yr[2];
      readout(yr, cf, sHs, l);
      const f32x4 rr = *reinterpret_cast<const f32x4*>(tok + kRr * 64 + 16 * w + 4 * q4);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[tp][r] += rr[r] * yr[tp][r];
    }
    // the partial output of the run (bf16) into out
    {
      float v[2][4];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[tp][r] = y[tp][r];
      tile_rows_to_lds(slot, v, l);
      const int64_t t = t0 + 16 * w + (l >> 2);
      if (t < a.L)
        *reinterpret_cast<uint4*>(a.out + (b * a.L + t) * (a.H * P) + h * P + 8 * (l & 3)) =
            *reinterpret_cast<const uint4*>(slot + (l >> 2) * P + 8 * (l & 3));
    }
    const float eS = ex(tok[kS * 64 + 63]);
    if (kRev) state_update(G, eS, sBT, sXWr, w, l);
    if (kFwd) state_update(F, 1.0f, sBT, sXWf, w, l);
    if (tid == 0) a.tau[item * a.rpc + k] = tau;
    tau *= eS;
    if (w == 0 && st + 1 < nrun) token_prep(sTok[(st + 1) & 1], pdt, (sub0 + k - 1) * Q + l < a.L, Ah, bias, l);
    pdt = pdt2;
  }
  if (kFwd) state_store(F, a.S + (item * 2 + 0) * kSF, w, l);
  if (kRev) state_store(G, a.S + (item * 2 + 1) * kSF, w, l);
  if (tid == 0) a.Pc[item] = tau;
}

// ---------------------------------------------------------------------------
// k_ssd_carry: chunk-local states -> states entering each chunk (in place).
// One thread per (batch, head, state element); sequential over chunks.  In
// block decoding the forward chain starts from the cached state h_in and its
// value after the last chunk is the new cache h_out (both [batch, H, P, N]);
// each thread reads and writes only its own element, so h_out may be h_in.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ssd_carry(float* S, const float* Pc, int64_t batch, int64_t H,
                                                   int64_t nchunk, int dirs, const float* h_in, float* h_out) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t e = gid % kSF, bh = gid / kSF;
  if (bh >= batch * H) return;
  const int64_t b = bh / H, h = bh % H;
  if (dirs & 1) {
    // element e of the tile layout [nb][tp][lane][r] is state n of channel p
    const int64_t r = e % 4, ln = (e / 4) % 64, tp = (e / 256) % 2, nb = e / 512;
    const int64_t n = 16 * nb + 4 * (ln / 16) + r, p = 16 * tp + ln % 16;
    const int64_t hidx = ((b * H + h) * P + p) * N + n;
    float acc = h_in ? h_in[hidx] : 0.0f;
    for (int64_t c = 0; c < nchunk; ++c) {
      const int64_t item = (b * nchunk + c) * H + h;
      float* p_s = S + (item * 2 + 0) * kSF + e;
      const float t = *p_s;
      *p_s = acc;
      acc = Pc[item] * acc + t;
    }
    if (h_out) h_out[hidx] = acc;
  }
  if (dirs & 2) {
    float acc = 0.0f;
    for (int64_t c = nchunk - 1; c >= 0; --c) {
      const int64_t item = (b * nchunk + c) * H + h;
      float* p = S + (item * 2 + 1) * kSF + e;
      const float t = *p;
      *p = acc;
      acc = Pc[item] * acc + t;
    }
  }
}

// ---------------------------------------------------------------------------
// k_ssd_fsweep: left to right over a chunk's runs; same wavefront roles as the
// reverse sweep.  DIRS bit 0 = forward, bit 1 = reverse.
// ---------------------------------------------------------------------------
template <int DIRS>
__global__ __launch_bounds__(kThreads, 2) void k_ssd_fsweep(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXW[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sHs[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sHg[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sZ[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) uint16_t sY[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) float sTok[2][kTokRows * 64];
  constexpr bool kFwd = DIRS & 1, kRev = DIRS & 2;
  constexpr float kDiag = (kFwd && kRev) ? 2.0f : 1.0f;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  int64_t b, c, h;
  decode_item(a, b, c, h);
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float Dfac = a.D ? a.D[h] * kDiag : 0.0f;
  const int64_t sub0 = c * a.rpc;
  const int64_t nrun = a.nsub - sub0 < a.rpc ? a.nsub - sub0 : a.rpc;
  const int64_t item = (b * a.nchunk + c) * a.H + h;
  const int64_t HP = a.H * P;
  uint16_t* zslot = sZ + w * 16 * P;
  uint16_t* yslot = sY + w * 16 * P;
  State H;
  if (kFwd) state_load(H, a.S + (item * 2 + 0) * kSF, w, l);
  if (kRev) {
    // the reverse state entering the chunk from the right is fixed for the whole chunk
    State Gin;
    state_load(Gin, a.S + (item * 2 + 1) * kSF, w, l);
    state_to_lds(Gin, sHg, w, l);
  }

  u32x4 pc[4], pbt[4];
  uint4 px, pz, py;
  float ptau = 0.0f;
  uint16_t pdt = 0, pdt2 = 0;  // step sizes two steps ahead, as in the reverse sweep
  auto issue = [&](int64_t k) {
    const int64_t sub = sub0 + k, t0 = sub * Q;
    if (w == 0 && k + 1 < nrun) pdt2 = load_dt(a, b, t0 + Q, h, l);
    const int64_t tile = (b * a.nsub + sub) * static_cast<int64_t>(Q * N);
    const u32x4* b4 = reinterpret_cast<const u32x4*>(a.bt + tile);
    load_cfrag(pc, a.cp + tile, w, l);
    if (kFwd) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pbt[i] = b4[tid + kThreads * i];
    }
    px = load_act(a.x, a, b, t0, h, tid);
    const int q = 64 * w + l;  // this wavefront's rows 16w..16w+15 (q/4 = 16w + l/4)
    py = load_act(a.out, a, b, t0, h, q);
    if (a.gate) pz = load_act(a.z, a, b, t0, h, q);
    if (kRev) ptau = a.tau[item * a.rpc + k];
  };
  if (w == 0) pdt = load_dt(a, b, sub0 * Q, h, l);
  issue(0);
  if (w == 0) token_prep(sTok[0], pdt, sub0 * Q + l < a.L, Ah, bias, l);
  pdt = pdt2;
  // a run's output is stored at the start of the next step's computation, just before that step's
  // loads are issued: the store has a whole step to complete before the wait for those loads
  uint4 pend = make_uint4(0, 0, 0, 0);

  for (int64_t k = 0; k < nrun; ++k) {
    const int64_t t0 = (sub0 + k) * Q;
    const float* tok = sTok[k & 1];
    bf16x8 cf[4];
    __syncthreads();
    // ---- commit the prefetched registers ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + kThreads * i;
      if (kFwd) *reinterpret_cast<u32x4*>(sBT + sw128(ci >> 3, ci & 7)) = pbt[i];
      cf[i] = __builtin_bit_cast(bf16x8, pc[i]);
    }
    put_xt(sXT, px, tid, nullptr, 1.0f);
    if (kFwd) put_xt(sXW, px, tid, tok + kWf * 64, 1.0f);
    *reinterpret_cast<uint4*>(yslot + (l >> 2) * P + 8 * (l & 3)) = py;
    if (a.gate) *reinterpret_cast<uint4*>(zslot + (l >> 2) * P + 8 * (l & 3)) = pz;
    const float tau_run = ptau;
    if (kFwd) state_to_lds(H, sHs, w, l);
    __syncthreads();
    if (k > 0) store_run_row(a.out, b, a.L, HP, t0 - Q, h, 16 * w + (l >> 2), l & 3, pend);
    if (k + 1 < nrun) issue(k + 1);

    // ---- compute ----
    f32x4 y[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[tp][r] = bf(yslot[(4 * q4 + r) * P + 16 * tp + l16]);
    if (kFwd) {
      f32x4 yf[2];
      readout(yf, cf, sHs, l);
      const f32x4 rf = *reinterpret_cast<const f32x4*>(tok + kRf * 64 + 16 * w + 4 * q4);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[tp][r] += rf[r] * yf[tp][r];
    }
    if (kRev) {
      f32x4 yg[2];
      readout(yg, cf, sHg, l);
      const f32x4 rr = *reinterpret_cast<const f32x4*>(tok + kRr * 64 + 16 * w + 4 * q4);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[tp][r] += (tau_run * rr[r]) * yg[tp][r];
    }
    // skip term and gate
    float o[2][4];
    const int i0 = 16 * w + 4 * q4;
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int p = 16 * tp + l16;
      const uint2 xv = *reinterpret_cast<const uint2*>(sXT + sw128(p, i0 >> 3) + (i0 & 7));
      const float xs[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xffff0000u),
                           __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xffff0000u)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[tp][r] = y[tp][r] + Dfac * xs[r];
        if (a.gate) o[tp][r] *= silu_f32(bf(zslot[(4 * q4 + r) * P + p]));
      }
    }
    tile_rows_to_lds(yslot, o, l);
    pend = *reinterpret_cast<const uint4*>(yslot + (l >> 2) * P + 8 * (l & 3));
    if (kFwd) state_update(H, ex(tok[kS * 64 + 63]), sBT, sXW, w, l);
    if (w == 0 && k + 1 < nrun) token_prep(sTok[(k + 1) & 1], pdt, (sub0 + k + 1) * Q + l < a.L, Ah, bias, l);
    pdt = pdt2;
  }
  store_run_row(a.out, b, a.L, HP, (sub0 + nrun - 1) * Q, h, 16 * w + (l >> 2), l & 3, pend);
}

// ---------------------------------------------------------------------------
// k_ssd_block: one block of block-cache decoding of at most Q tokens (one run)
// for one (batch, head) per workgroup, in a single kernel.  The run's C B^T,
// B^T and per-token terms are formed here instead of by the tiling kernel; out
// = the intra-run products of both directions (the reverse direction starts
// from zero after the block), the readout of the cached forward state, the
// skip term and the gate; the new cache = the cached state decayed over the
// block plus the block's own update.  Wavefront w owns output rows 16w..16w+15
// and state row blocks 2w, 2w + 1, as in the sweeps.  The cache is read and
// written in the caller's layout [batch, H, P, N]; each element is read and
// written by the same lane, so h_out may be h_in.  The products whose operand
// is not exact in bf16 (the decay-weighted C B^T of the intra-block product,
// the cached state in its readout, the weighted x of the cache update) take
// that operand as a rounded value and its rounding residual, two products
// each, so the cache and the output before its own rounding keep fp32-level
// accuracy (2^-16 of each term) over any number of chained blocks.
// ---------------------------------------------------------------------------
template <int DIRS>
__global__ __launch_bounds__(kThreads, 2) void k_ssd_block(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBs[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sCs[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXW[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXWr[P * Q];  // rounding residuals of sXW
  __shared__ __attribute__((aligned(16))) uint16_t sHs[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sHr[P * N];   // rounding residuals of sHs
  __shared__ __attribute__((aligned(16))) uint16_t sZ[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) uint16_t sY[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) float sTok[kTokRows * 64];
  constexpr bool kFwd = DIRS & 1, kRev = DIRS & 2;
  constexpr float kDiag = (kFwd && kRev) ? 2.0f : 1.0f;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  const int64_t h = blockIdx.x % a.H, b = blockIdx.x / a.H;
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float Dfac = a.D ? a.D[h] * kDiag : 0.0f;
  const int64_t HP = a.H * P;
  uint16_t* zslot = sZ + w * 16 * P;
  uint16_t* yslot = sY + w * 16 * P;

  // 1. the block's B and C rows (zero past its end), the head's x, z and step sizes, and the cache
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int j = ci >> 4, cc = ci & 15;
    uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
    if (j < a.L) {
      vb = *reinterpret_cast<const uint4*>(a.B + (b * a.L + j) * N + 8 * cc);
      vc = *reinterpret_cast<const uint4*>(a.C + (b * a.L + j) * N + 8 * cc);
    }
    *reinterpret_cast<uint4*>(sBs + sw256(j, cc)) = vb;
    *reinterpret_cast<uint4*>(sCs + sw256(j, cc)) = vc;
  }
  const uint4 px = load_act(a.x, a, b, 0, h, tid);
  if (a.gate) *reinterpret_cast<uint4*>(zslot + (l >> 2) * P + 8 * (l & 3)) = load_act(a.z, a, b, 0, h, 64 * w + l);
  State H;
  state_zero(H);
  if (kFwd && a.h_in) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * (2 * w + i) + 4 * q4 + r, p = 16 * tp + l16;
          H.t[i][tp][r] = a.h_in[((b * a.H + h) * P + p) * N + n];
        }
  }
  if (w == 0) token_prep(sTok, load_dt(a, b, 0, h, l), l < a.L, Ah, bias, l);
  __syncthreads();

  // 2. B^T rows (the state update's operand), this wavefront's rows of C B^T, x tiles, the cache as bf16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int n = ci >> 3, jc = ci & 7;
    uint32_t w2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = 8 * jc + 2 * e;
      w2[e] = static_cast<uint32_t>(sBs[sw256(j0, n >> 3) + (n & 7)]) |
              (static_cast<uint32_t>(sBs[sw256(j0 + 1, n >> 3) + (n & 7)]) << 16);
    }
    *reinterpret_cast<uint4*>(sBT + sw128(n, jc)) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
  }
  bf16x8 cf[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cf[k] = lds8(sCs, sw256(16 * w + l16, 4 * k + q4));
  f32x4 gcur[4];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    f32x4 acc = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = mfma(lds8(sBs, sw256(16 * tj + l16, 4 * k + q4)), cf[k], acc);
    gcur[tj] = acc;
  }
  const float* tok = sTok;
  put_xt(sXT, px, tid, nullptr, 1.0f);
  if (kFwd) put_xt_split(sXW, sXWr, px, tid, tok + kWf * 64);
  if (kFwd) state_to_lds_split(H, sHs, sHr, w, l);
  __syncthreads();

  // 3. out.  W = mask o (C B^T) o delta_j for rows i = 16w + l16 as the A operand, k-slots permuted as in
  // the reverse sweep: slot e < 4 -> j = 32k2 + 4q4 + e, slot e >= 4 -> j = 32k2 + 16 + 4q4 + e - 4
  const int i = 16 * w + l16;
  const float si = tok[kS * 64 + i], ei = tok[kE * 64 + i];
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    const int j0 = 16 * tj + 4 * q4;
    const f32x4 sj = *reinterpret_cast<const f32x4*>(tok + kS * 64 + j0);
    const f32x4 ej = *reinterpret_cast<const f32x4*>(tok + kE * 64 + j0);
    const f32x4 dj = *reinterpret_cast<const f32x4*>(tok + kDl * 64 + j0);
    mask_block<kFwd, kRev>(gcur[tj], tj, __builtin_amdgcn_readfirstlane(w), i, j0, si, ei, sj, ej, dj, kDiag);
  }
  f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    // the weights as rounded values and residuals (x is exact in bf16)
    bf16x8 wa, wr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t h0 = to_bf(gcur[2 * k2][r]), h1 = to_bf(gcur[2 * k2 + 1][r]);
      wa[r] = __builtin_bit_cast(__bf16, h0);
      wa[4 + r] = __builtin_bit_cast(__bf16, h1);
      wr[r] = __builtin_bit_cast(__bf16, bf_rest(gcur[2 * k2][r], h0));
      wr[4 + r] = __builtin_bit_cast(__bf16, bf_rest(gcur[2 * k2 + 1][r], h1));
    }
    const int jlo = 32 * k2 + 4 * q4;
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int p = 16 * tp + l16;
      const uint2 lo = *reinterpret_cast<const uint2*>(sXT + sw128(p, jlo >> 3) + (jlo & 7));
      const uint2 hi = *reinterpret_cast<const uint2*>(sXT + sw128(p, (jlo + 16) >> 3) + (jlo & 7));
      const bf16x8 xb = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      y[tp] = mfma(wr, xb, mfma(wa, xb, y[tp]));
    }
  }
  if (kFwd) {
    f32x4 yf[2], yr[2];
    readout(yf, cf, sHs, l);
    readout(yr, cf, sHr, l);
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) yf[tp] += yr[tp];
    const f32x4 rf = *reinterpret_cast<const f32x4*>(tok + kRf * 64 + 16 * w + 4 * q4);
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[tp][r] += rf[r] * yf[tp][r];
  }
  float o[2][4];
  const int i0 = 16 * w + 4 * q4;
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    const int p = 16 * tp + l16;
    const uint2 xv = *reinterpret_cast<const uint2*>(sXT + sw128(p, i0 >> 3) + (i0 & 7));
    const float xs[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xffff0000u),
                         __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xffff0000u)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o[tp][r] = y[tp][r] + Dfac * xs[r];
      if (a.gate) o[tp][r] *= silu_f32(bf(zslot[(4 * q4 + r) * P + p]));
    }
  }
  tile_rows_to_lds(yslot, o, l);
  {
    const int64_t t = 16 * w + (l >> 2);
    if (t < a.L)
      *reinterpret_cast<uint4*>(a.out + (b * a.L + t) * HP + h * P + 8 * (l & 3)) =
          *reinterpret_cast<const uint4*>(yslot + (l >> 2) * P + 8 * (l & 3));
  }

  // 4. the new cache: the cached state decayed over the block plus the block's update
  if (kFwd && a.h_out) {
    state_update(H, ex(tok[kS * 64 + 63]), sBT, sXW, w, l);
    state_update(H, 1.0f, sBT, sXWr, w, l);
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * (2 * w + i2) + 4 * q4 + r, p = 16 * tp + l16;
          a.h_out[((b * a.H + h) * P + p) * N + n] = H.t[i2][tp][r];
        }
  }
}

// ---------------------------------------------------------------------------
// One-direction Mamba-2 layers (the paper's untied directions: each direction is its own layer), with the
// layer's short convolution optionally applied as the inputs are loaded.
//
// x, B and C are columns of one projection stream of a.xs elements per token.  With a.cw set, the stream
// first goes through the width-4 depthwise convolution of its channel and the SiLU: causal for the forward
// layer, anti-causal for the reverse one (the forward layer applied to the flipped sequence); the result is
// rounded to bf16 as if it had been stored between two passes.  A one-direction scan needs no partial
// output between passes:
//   k_ssd1_stage    per run: B, C (convolved) into the run tiles: C, B^T and C B^T;
//   k_ssd1_summary  per (chunk, head), in the scan's direction over the runs: the state update only, giving
//                   the chunk's end state from zero and the product of abar over the chunk;
//   k_ssd_carry     the chunk maps across the sequence (the bidirectional pass's kernel, one direction);
//   k_ssd1_walk     per (chunk, head), in the scan's direction: the intra-run product of the one-direction
//                   mask, the readout of the running state, the skip term and the gate, the store, and the
//                   state update.
// DIR = 1: forward (runs left to right), 2: reverse (right to left).
// ---------------------------------------------------------------------------

// One stream channel of a run through the convolution: rows of the run's 64 tokens t0 .. t0 + 63 and the
// 3-token halo (before them for the causal filter, after them for the anti-causal one), zero outside the
// sequence; every load is issued from a clamped in-bounds row and the value selected afterwards.
template <int DIR, int NT>
__device__ __forceinline__ void conv_rows(const uint16_t* col, int64_t xs, int64_t L, int64_t tfirst,
                                          uint16_t (&r)[NT + 3]) {
#pragma unroll
  for (int i = 0; i < NT + 3; ++i) {
    const int64_t t = tfirst + i;
    const int64_t tc = t < 0 ? 0 : (t >= L ? L - 1 : t);
    const uint16_t v = col[tc * xs];
    r[i] = (t >= 0 && t < L) ? v : static_cast<uint16_t>(0);
  }
}

// NT outputs from the rows of conv_rows (r[0] is row tfirst): causal out[t] = silu(b + sum_k w[k] u[t-3+k])
// with tfirst = t0 - 3, anti-causal out[t] = silu(b + sum_k w[k] u[t+3-k]) with tfirst = t0; rounded to
// bf16; tokens at or past L give 0 (padding of the last run).
template <int DIR, int NT>
__device__ __forceinline__ void conv_outputs(const uint16_t (&r)[NT + 3], const float (&w)[4], float bias,
                                             int64_t t0, int64_t L, uint16_t (&o)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float acc = bias;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(w[k], bf(DIR == 1 ? r[i + k] : r[i + 3 - k]), acc);
    o[i] = (t0 + i < L) ? to_bf(silu_f32(acc)) : static_cast<uint16_t>(0);
  }
}

// The channel's conv taps and bias (stream channel ch).
__device__ __forceinline__ void conv_taps(const Args& a, int64_t ch, float (&w)[4], float& bias) {
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = a.cw[ch * 4 + k];
  bias = a.cb ? a.cb[ch] : 0.0f;
}

// k_ssd1_stage: one workgroup per (run, batch element).  With the convolution, thread n < 128 convolves B
// channel n and thread 128 + n C channel n over the run's 64 tokens into LDS; without it the rows are copied
// (zero past the sequence end).  Then, as in k_ssd_stage: the C tile, B^T and C B^T.
template <int DIR, bool CONV>
__global__ __launch_bounds__(kThreads) void k_ssd1_stage(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBs[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sCs[Q * N];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  const int64_t sub = blockIdx.x, b = blockIdx.y;
  const int64_t t0 = sub * Q;
  const int64_t HP = a.H * P;
  const int64_t tile = (b * a.nsub + sub) * static_cast<int64_t>(Q * N);
  const uint16_t* rows = a.x + b * a.L * a.xs;  // this batch element's stream
  if (CONV) {
    const int n = tid & (N - 1);
    const bool isC = tid >= N;
    const int64_t ch = HP + (isC ? N : 0) + n;
    float wv[4], bias;
    conv_taps(a, ch, wv, bias);
    uint16_t* dst = isC ? sCs : sBs;
    // 64 tokens in 4 groups of 16, so that the rows of one group stay in registers
#pragma unroll 1
    for (int g = 0; g < Q / 16; ++g) {
      uint16_t r[16 + 3], o[16];
      conv_rows<DIR, 16>(rows + ch, a.xs, a.L, t0 + 16 * g + (DIR == 1 ? -3 : 0), r);
      conv_outputs<DIR, 16>(r, wv, bias, t0 + 16 * g, a.L, o);
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[sw256(16 * g + i, n >> 3) + (n & 7)] = o[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + kThreads * i;
      const int j = ci >> 4, cc = ci & 15;
      uint4 vb = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
      if (t0 + j < a.L) {
        vb = *reinterpret_cast<const uint4*>(rows + (t0 + j) * a.xs + HP + 8 * cc);
        vc = *reinterpret_cast<const uint4*>(rows + (t0 + j) * a.xs + HP + N + 8 * cc);
      }
      *reinterpret_cast<uint4*>(sBs + sw256(j, cc)) = vb;
      *reinterpret_cast<uint4*>(sCs + sw256(j, cc)) = vc;
    }
  }
  __syncthreads();
  // the C tile (rows of N states per token)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int j = ci >> 4, cc = ci & 15;
    *reinterpret_cast<uint4*>(a.cp + tile + j * N + 8 * cc) = *reinterpret_cast<const uint4*>(sCs + sw256(j, cc));
  }
  // B^T rows n, 8 tokens per 16-byte chunk
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = tid + kThreads * i;
    const int n = ci >> 3, jc = ci & 7;
    uint32_t w2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = 8 * jc + 2 * e;
      w2[e] = static_cast<uint32_t>(sBs[sw256(j0, n >> 3) + (n & 7)]) |
              (static_cast<uint32_t>(sBs[sw256(j0 + 1, n >> 3) + (n & 7)]) << 16);
    }
    *reinterpret_cast<uint4*>(a.bt + tile + n * Q + 8 * jc) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
  }
  // C B^T: wavefront w forms the 4 tiles of row block ib = w
  bf16x8 cf[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cf[k] = lds8(sCs, sw256(16 * w + l16, 4 * k + q4));
  float* gout = a.g + (b * a.nsub + sub) * static_cast<int64_t>(Q * Q);
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    f32x4 acc = zero4();
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = mfma(lds8(sBs, sw256(16 * tj + l16, 4 * k + q4)), cf[k], acc);
    *reinterpret_cast<f32x4*>(gout + ((w * 4 + tj) * 64 + l) * 4) = acc;
  }
}

// A run's x for one head, the way the walks consume it.  With the convolution: thread tid owns channel
// c = tid % 32 of the head and tokens 8g .. 8g + 7 of the run (g = tid / 32): it loads those 8 rows and the
// 3-token halo of its channel (raw, 11 values), convolves them at commit time and writes one 16-byte chunk
// of the channel-major LDS tiles.  Without it: 16 bytes (token tid / 4, channels 8(tid % 4) .. + 7) as in
// the bidirectional sweeps.
template <int DIR, bool CONV>
struct XRun;

// Rows of a run's window for the convolution: the run's 64 tokens and the 3-token halo (before them for the
// causal filter, after them for the anti-causal one).
constexpr int kWinRows = Q + 3;

template <int DIR>
struct XRun<DIR, true> {
  // The window's rows of the head's 32 x channels (64 bytes each) are brought into LDS (sRaw, double
  // buffered) by direct-to-LDS buffer loads, 16 bytes per lane: chunk q = 4 row + part lands at byte 16 q.
  // The resource starts at channel h P of the batch element's first token and ends with its last token, so
  // the rows before the sequence (negative offsets wrap to huge ones) and after it are out of range and read
  // as zero.  The compiler does not track these loads: the walk waits for them (vmcnt 0) before the barrier
  // that precedes their use.
  uint16_t* sRaw;  // [2][kWinRows * P]
  __device__ __forceinline__ void load(const Args& a, int64_t b, int64_t t0, int64_t h, int tid, int buf) {
    const int64_t tfirst = t0 + (DIR == 1 ? -3 : 0);
    const uint16_t* base = a.x + b * a.L * a.xs + h * P;
    const int64_t bytes = (a.L * a.xs - h * P) * 2;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
    uint16_t* dst = sRaw + buf * (kWinRows * P);
    const int w = tid >> 6, lane = tid & 63;
    // chunks 64 w + lane (rows 16 w .. 16 w + 15), then chunks 256 .. 267 (the last 3 rows) by wavefront 0
    for (int pass = 0; pass < 2; ++pass) {
      const int q = pass == 0 ? 64 * w + lane : 256 + lane;
      if (pass == 1 && (w != 0 || lane >= 4 * kWinRows - 256)) break;
      const int row = q >> 2, part = q & 3;
      const int32_t off = static_cast<int32_t>((tfirst + row) * a.xs * 2) + part * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (q - lane) * 8),
                                               16, static_cast<uint32_t>(off), 0, 0, 0);
    }
  }
  // the convolution of the window in sRaw[buf]: thread tid convolves channel c = tid % 32 over tokens
  // 8 g .. 8 g + 7 (g = tid / 32); returns that chunk of the x tile (8 bf16 values, token order)
  __device__ __forceinline__ uint4 conv(const float (&w)[4], float bias, int64_t t0, int64_t L, int tid, int buf) const {
    const int c = tid & 31, g = tid >> 5;
    const uint16_t* src = sRaw + buf * (kWinRows * P);
    uint16_t r[8 + 3], o[8];
#pragma unroll
    for (int i = 0; i < 11; ++i) r[i] = src[(8 * g + i) * P + c];
    conv_outputs<DIR, 8>(r, w, bias, t0 + 8 * g, L, o);
    return make_uint4(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16),
                      o[4] | (static_cast<uint32_t>(o[5]) << 16), o[6] | (static_cast<uint32_t>(o[7]) << 16));
  }
  // this thread's chunk v of the x tile into the channel-major tile dst (sXT's layout)
  __device__ __forceinline__ void put(uint16_t* dst, uint4 v, int tid) const {
    *reinterpret_cast<uint4*>(dst + sw128(tid & 31, tid >> 5)) = v;
  }
  // this thread's chunk v weighted per token (weights wtok[j] * wscale) into dst
  __device__ __forceinline__ void weight(uint16_t* dst, uint4 v, const float* wtok, float wscale, int tid) const {
    const int c = tid & 31, g = tid >> 5;
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(in[e] << 16) * (wtok[8 * g + 2 * e] * wscale);
      const float hi = __uint_as_float(in[e] & 0xffff0000u) * (wtok[8 * g + 2 * e + 1] * wscale);
      q[e] = static_cast<uint32_t>(to_bf(lo)) | (static_cast<uint32_t>(to_bf(hi)) << 16);
    }
    *reinterpret_cast<uint4*>(dst + sw128(c, g)) = make_uint4(q[0], q[1], q[2], q[3]);
  }
};

template <int DIR>
struct XRun<DIR, false> {
  uint4 px;
  __device__ __forceinline__ void load(const Args& a, int64_t b, int64_t t0, int64_t h, int tid, int) {
    const int j = tid >> 2, pc = tid & 3;
    px = (t0 + j >= a.L) ? make_uint4(0, 0, 0, 0)
                         : *reinterpret_cast<const uint4*>(a.x + (b * a.L + t0 + j) * a.xs + h * P + 8 * pc);
  }
  __device__ __forceinline__ void commit(uint16_t* sXT, uint16_t* sXW, const float* wtok, float wscale,
                                         const float (&)[4], float, int64_t, int64_t, int tid, int) const {
    if (sXT) put_xt(sXT, px, tid, nullptr, 1.0f);
    if (sXW) put_xt(sXW, px, tid, wtok, wscale);
  }
};

// k_ssd1_summary: one workgroup per (batch, chunk, head), over the chunk's runs in the scan's direction:
// state <- e^{S_run} state + B^T (weighted x), from zero.  The forward layer's end state (slot 0 of the
// chunk's state pair) weights token j by e^{S_run - s_j} delta_j, the reverse layer's (slot 1) by e^{e_j}
// delta_j.  Also the product of abar over the chunk.
template <int DIR, bool CONV>
__global__ __launch_bounds__(kThreads, 2) void k_ssd1_summary(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXW[P * Q];
  __shared__ __attribute__((aligned(16))) float sTok[2][kTokRows * 64];
  // with the convolution: the raw windows, double buffered (the next run's arrives during this run's step)
  __shared__ __attribute__((aligned(16))) uint16_t sRaw[CONV ? 2 * kWinRows * P : 8];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int64_t b, c, h;
  decode_item(a, b, c, h);
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const int64_t sub0 = c * a.rpc;
  const int64_t nrun = a.nsub - sub0 < a.rpc ? a.nsub - sub0 : a.rpc;
  const int64_t item = (b * a.nchunk + c) * a.H + h;
  float cw[4] = {0.f, 0.f, 0.f, 0.f}, cbias = 0.0f;
  if (CONV) conv_taps(a, h * P + (tid & 31), cw, cbias);
  State S;
  state_zero(S);
  float prod = 1.0f;  // product of abar over the runs done
  u32x4 pbt[4];
  XRun<DIR, CONV> xr;
  if constexpr (CONV) xr.sRaw = sRaw;
  uint16_t pdt = 0, pdt2 = 0;  // step sizes two steps ahead
  auto run_of = [&](int64_t st) { return DIR == 1 ? st : nrun - 1 - st; };
  auto issue = [&](int64_t st) {
    const int64_t sub = sub0 + run_of(st);
    if (w == 0 && st + 1 < nrun) pdt2 = load_dt(a, b, (sub0 + run_of(st + 1)) * Q, h, l);
    const u32x4* b4 = reinterpret_cast<const u32x4*>(a.bt + (b * a.nsub + sub) * static_cast<int64_t>(Q * N));
#pragma unroll
    for (int i = 0; i < 4; ++i) pbt[i] = b4[tid + kThreads * i];
    xr.load(a, b, sub * Q, h, tid, static_cast<int>(st & 1));
  };
  if (w == 0) pdt = load_dt(a, b, (sub0 + run_of(0)) * Q, h, l);
  issue(0);
  if (w == 0) token_prep(sTok[0], pdt, (sub0 + run_of(0)) * Q + l < a.L, Ah, bias, l);
  pdt = pdt2;
  for (int64_t st = 0; st < nrun; ++st) {
    const int64_t t0 = (sub0 + run_of(st)) * Q;
    const float* tok = sTok[st & 1];
    if (CONV) wait_vmem();  // this run's window, brought into LDS by the last step's direct loads
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(sBT + sw128(ci >> 3, ci & 7)) = pbt[i];
    }
    if constexpr (CONV) {
      xr.weight(sXW, xr.conv(cw, cbias, t0, a.L, tid, static_cast<int>(st & 1)), tok + (DIR == 1 ? kWf : kWr) * 64,
                1.0f, tid);
    } else {
      xr.commit(nullptr, sXW, tok + (DIR == 1 ? kWf : kWr) * 64, 1.0f, cw, cbias, t0, a.L, tid, 0);
    }
    __syncthreads();
    if (st + 1 < nrun) issue(st + 1);
    const float eS = ex(tok[kS * 64 + 63]);
    state_update(S, eS, sBT, sXW, w, l);
    prod *= eS;
    if (w == 0 && st + 1 < nrun)
      token_prep(sTok[(st + 1) & 1], pdt, (sub0 + run_of(st + 1)) * Q + l < a.L, Ah, bias, l);
    pdt = pdt2;
  }
  state_store(S, a.S + (item * 2 + (DIR == 1 ? 0 : 1)) * kSF, w, l);
  if (tid == 0) a.Pc[item] = prod;
}

// k_ssd1_walk: one workgroup per (batch, chunk, head), over the chunk's runs in the scan's direction, from
// the state entering the chunk (the carry pass's output).  Wavefront w owns output rows 16w .. 16w + 15 and
// state row blocks 2w, 2w + 1, as in the bidirectional sweeps.
template <int DIR, bool CONV>
__global__ __launch_bounds__(kThreads, 2) void k_ssd1_walk(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sXW[P * Q];
  __shared__ __attribute__((aligned(16))) uint16_t sHs[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sZ[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) uint16_t sY[4 * 16 * P];
  __shared__ __attribute__((aligned(16))) float sTok[2][kTokRows * 64];
  // with the convolution: the raw windows, double buffered (the next run's arrives during this run's step);
  // each is convolved in the commit phase, whose VALU slots are otherwise mostly idle
  __shared__ __attribute__((aligned(16))) uint16_t sRaw[CONV ? 2 * kWinRows * P : 8];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q4 = l >> 4, l16 = l & 15;
  int64_t b, c, h;
  decode_item(a, b, c, h);
  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float Dfac = a.D ? a.D[h] : 0.0f;
  const int64_t sub0 = c * a.rpc;
  const int64_t nrun = a.nsub - sub0 < a.rpc ? a.nsub - sub0 : a.rpc;
  const int64_t item = (b * a.nchunk + c) * a.H + h;
  const int64_t HP = a.H * P;
  uint16_t* zslot = sZ + w * 16 * P;
  uint16_t* yslot = sY + w * 16 * P;
  float cw[4] = {0.f, 0.f, 0.f, 0.f}, cbias = 0.0f;
  if (CONV) conv_taps(a, h * P + (tid & 31), cw, cbias);
  State H;
  state_load(H, a.S + (item * 2 + (DIR == 1 ? 0 : 1)) * kSF, w, l);

  u32x4 pc[4], pbt[4];
  f32x4 pg[4];
  uint4 pz;
  XRun<DIR, CONV> xr;
  if constexpr (CONV) xr.sRaw = sRaw;
  uint16_t pdt = 0, pdt2 = 0;
  auto run_of = [&](int64_t st) { return DIR == 1 ? st : nrun - 1 - st; };
  auto issue = [&](int64_t st) {
    const int64_t sub = sub0 + run_of(st), t0 = sub * Q;
    if (w == 0 && st + 1 < nrun) pdt2 = load_dt(a, b, (sub0 + run_of(st + 1)) * Q, h, l);
    const int64_t tile = (b * a.nsub + sub) * static_cast<int64_t>(Q * N);
    const u32x4* b4 = reinterpret_cast<const u32x4*>(a.bt + tile);
    load_cfrag(pc, a.cp + tile, w, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) pbt[i] = b4[tid + kThreads * i];
    const float* gg = a.g + (b * a.nsub + sub) * static_cast<int64_t>(Q * Q);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) pg[tj] = *reinterpret_cast<const f32x4*>(gg + ((w * 4 + tj) * 64 + l) * 4);
    xr.load(a, b, t0, h, tid, static_cast<int>(st & 1));
    if (a.gate) pz = load_act(a.z, a, b, t0, h, 64 * w + l);
  };
  if (w == 0) pdt = load_dt(a, b, (sub0 + run_of(0)) * Q, h, l);
  issue(0);
  if (w == 0) token_prep(sTok[0], pdt, (sub0 + run_of(0)) * Q + l < a.L, Ah, bias, l);
  pdt = pdt2;
  // a run's output is stored at the start of the next step's computation, before that step's loads
  uint4 pend = make_uint4(0, 0, 0, 0);
  int64_t t_pend = 0;

  for (int64_t st = 0; st < nrun; ++st) {
    const int64_t t0 = (sub0 + run_of(st)) * Q;
    const float* tok = sTok[st & 1];
    uint16_t* xt = sXT;
    bf16x8 cf[4];
    f32x4 gcur[4];
    if (CONV) wait_vmem();  // this run's window, brought into LDS by the last step's direct loads
    __syncthreads();
    // ---- commit the prefetched registers ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(sBT + sw128(ci >> 3, ci & 7)) = pbt[i];
      cf[i] = __builtin_bit_cast(bf16x8, pc[i]);
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) gcur[tj] = pg[tj];
    if constexpr (CONV) {
      const uint4 xc = xr.conv(cw, cbias, t0, a.L, tid, static_cast<int>(st & 1));
      xr.put(sXT, xc, tid);
      xr.weight(sXW, xc, tok + (DIR == 1 ? kWf : kWr) * 64, 1.0f, tid);
    } else {
      xr.commit(sXT, sXW, tok + (DIR == 1 ? kWf : kWr) * 64, 1.0f, cw, cbias, t0, a.L, tid, 0);
    }
    if (a.gate) *reinterpret_cast<uint4*>(zslot + (l >> 2) * P + 8 * (l & 3)) = pz;
    state_to_lds(H, sHs, w, l);
    __syncthreads();
    if (st > 0) store_run_row(a.out, b, a.L, HP, t_pend, h, 16 * w + (l >> 2), l & 3, pend);
    if (st + 1 < nrun) issue(st + 1);

    // ---- compute ----
    // W = mask o (C B^T) o delta_j for rows i = 16w + l16, k-slots permuted as in the bidirectional sweeps;
    // the mask keeps one direction: forward e^{s_i - s_j} for j < i, reverse e^{e_j - e_i} for j > i, 1 on
    // the diagonal
    const int i = 16 * w + l16;
    const float si = tok[kS * 64 + i], ei = tok[kE * 64 + i];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int j0 = 16 * tj + 4 * q4;
      const f32x4 sj = *reinterpret_cast<const f32x4*>(tok + kS * 64 + j0);
      const f32x4 ej = *reinterpret_cast<const f32x4*>(tok + kE * 64 + j0);
      const f32x4 dj = *reinterpret_cast<const f32x4*>(tok + kDl * 64 + j0);
      mask_block<DIR == 1, DIR == 2>(gcur[tj], tj, __builtin_amdgcn_readfirstlane(w), i, j0, si, ei, sj, ej, dj,
                                     1.0f);
    }
    f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 wa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wa[r] = static_cast<__bf16>(gcur[2 * k2][r]);
        wa[4 + r] = static_cast<__bf16>(gcur[2 * k2 + 1][r]);
      }
      const int jlo = 32 * k2 + 4 * q4;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int p = 16 * tp + l16;
        const uint2 lo = *reinterpret_cast<const uint2*>(xt + sw128(p, jlo >> 3) + (jlo & 7));
        const uint2 hi = *reinterpret_cast<const uint2*>(xt + sw128(p, (jlo + 16) >> 3) + (jlo & 7));
        y[tp] = mfma(wa, __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y)), y[tp]);
      }
    }
    {
      // the running state's readout: forward e^{s_i} C_i . H, reverse e^{S - e_i} C_i . G
      f32x4 ys[2];
      readout(ys, cf, sHs, l);
      const f32x4 rs = *reinterpret_cast<const f32x4*>(tok + (DIR == 1 ? kRf : kRr) * 64 + 16 * w + 4 * q4);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[tp][r] += rs[r] * ys[tp][r];
    }
    // skip term and gate
    float o[2][4];
    const int i0 = 16 * w + 4 * q4;
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int p = 16 * tp + l16;
      const uint2 xv = *reinterpret_cast<const uint2*>(xt + sw128(p, i0 >> 3) + (i0 & 7));
      const float xs[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xffff0000u),
                           __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xffff0000u)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[tp][r] = y[tp][r] + Dfac * xs[r];
        if (a.gate) o[tp][r] *= silu_f32(bf(zslot[(4 * q4 + r) * P + p]));
      }
    }
    tile_rows_to_lds(yslot, o, l);
    pend = *reinterpret_cast<const uint4*>(yslot + (l >> 2) * P + 8 * (l & 3));
    t_pend = t0;
    state_update(H, ex(tok[kS * 64 + 63]), sBT, sXW, w, l);
    if (w == 0 && st + 1 < nrun)
      token_prep(sTok[(st + 1) & 1], pdt, (sub0 + run_of(st + 1)) * Q + l < a.L, Ah, bias, l);
    pdt = pdt2;
  }
  store_run_row(a.out, b, a.L, HP, t_pend, h, 16 * w + (l >> 2), l & 3, pend);
}

template <int DIR, bool CONV>
hipError_t launch_one_dir(const Args& a, int64_t batch, hipStream_t stream) {
  hipLaunchKernelGGL((k_ssd1_stage<DIR, CONV>), dim3(static_cast<unsigned>(a.nsub), static_cast<unsigned>(batch)),
                     dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned groups = static_cast<unsigned>(batch * a.nchunk * a.H);
  hipLaunchKernelGGL((k_ssd1_summary<DIR, CONV>), dim3(groups), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = batch * a.H * kSF;
  hipLaunchKernelGGL(k_ssd_carry, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, a.S,
                     a.Pc, batch, a.H, a.nchunk, DIR, nullptr, nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_ssd1_walk<DIR, CONV>), dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DIRS>
hipError_t launch_dirs(const Args& a, int64_t batch, hipStream_t stream, int stage) {
  const unsigned groups = static_cast<unsigned>(batch * a.nchunk * a.H);
  if (stage < 0 || stage == 1) {
    hipLaunchKernelGGL(k_ssd_rsweep<DIRS>, dim3(groups), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 2) {
    const int64_t threads = batch * a.H * kSF;
    hipLaunchKernelGGL(k_ssd_carry, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, a.S,
                       a.Pc, batch, a.H, a.nchunk, DIRS, a.h_in, a.h_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 3) {
    hipLaunchKernelGGL(k_ssd_fsweep<DIRS>, dim3(groups), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_ssd_block(const SsdArgs& in, int64_t batch, int64_t block_len, int64_t nheads, hipStream_t stream) {
  Args a{};
  a.x = static_cast<const uint16_t*>(in.x);
  a.dt = static_cast<const uint16_t*>(in.dt);
  a.A = in.A;
  a.B = static_cast<const uint16_t*>(in.B);
  a.C = static_cast<const uint16_t*>(in.C);
  a.D = in.D;
  a.z = static_cast<const uint16_t*>(in.z);
  a.dt_bias = in.dt_bias;
  a.out = static_cast<uint16_t*>(in.out);
  a.L = block_len;
  a.H = nheads;
  a.gate = (in.flags & kNoGate) ? 0 : 1;
  a.h_in = in.h_in;
  a.h_out = in.h_out;
  const dim3 grid(static_cast<unsigned>(batch * nheads));
  if (in.flags & kFwdOnly) {
    hipLaunchKernelGGL(k_ssd_block<1>, grid, dim3(kThreads), 0, stream, a);
  } else if (in.flags & kRevOnly) {
    hipLaunchKernelGGL(k_ssd_block<2>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_ssd_block<3>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_ssd_one_dir(const SsdArgs& in, const float* cw, const float* cb, int64_t xs, const SsdPlan& p,
                              void* workspace, int dir, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  Args a{};
  a.x = static_cast<const uint16_t*>(in.x);
  a.dt = static_cast<const uint16_t*>(in.dt);
  a.A = in.A;
  a.D = in.D;
  a.z = static_cast<const uint16_t*>(in.z);
  a.dt_bias = in.dt_bias;
  a.out = static_cast<uint16_t*>(in.out);
  a.L = p.seqlen;
  a.H = p.nheads;
  a.nsub = p.nsub;
  a.rpc = p.rpc;
  a.nchunk = p.nchunk;
  a.g = reinterpret_cast<float*>(ws + p.off_g);
  a.cp = reinterpret_cast<uint16_t*>(ws + p.off_cp);
  a.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
  a.S = reinterpret_cast<float*>(ws + p.off_s);
  a.Pc = reinterpret_cast<float*>(ws + p.off_p);
  a.tau = reinterpret_cast<float*>(ws + p.off_tau);
  a.gate = (in.flags & kNoGate) ? 0 : 1;
  a.xs = xs;
  a.cw = cw;
  a.cb = cb;
  if (dir == 1) return cw ? launch_one_dir<1, true>(a, p.batch, stream) : launch_one_dir<1, false>(a, p.batch, stream);
  return cw ? launch_one_dir<2, true>(a, p.batch, stream) : launch_one_dir<2, false>(a, p.batch, stream);
}

hipError_t launch_ssd(const SsdArgs& in, const SsdPlan& p, void* workspace, hipStream_t stream, int stage) {
  char* ws = static_cast<char*>(workspace);
  Args a{};
  a.x = static_cast<const uint16_t*>(in.x);
  a.dt = static_cast<const uint16_t*>(in.dt);
  a.A = in.A;
  a.B = static_cast<const uint16_t*>(in.B);
  a.C = static_cast<const uint16_t*>(in.C);
  a.D = in.D;
  a.z = static_cast<const uint16_t*>(in.z);
  a.dt_bias = in.dt_bias;
  a.out = static_cast<uint16_t*>(in.out);
  a.L = p.seqlen;
  a.H = p.nheads;
  a.nsub = p.nsub;
  a.rpc = p.rpc;
  a.nchunk = p.nchunk;
  a.g = reinterpret_cast<float*>(ws + p.off_g);
  a.cp = reinterpret_cast<uint16_t*>(ws + p.off_cp);
  a.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
  a.S = reinterpret_cast<float*>(ws + p.off_s);
  a.Pc = reinterpret_cast<float*>(ws + p.off_p);
  a.tau = reinterpret_cast<float*>(ws + p.off_tau);
  a.gate = (in.flags & kNoGate) ? 0 : 1;
  a.h_in = in.h_in;
  a.h_out = in.h_out;
  if (stage < 0 || stage == 0) {
    hipLaunchKernelGGL(k_ssd_stage, dim3(static_cast<unsigned>(p.nsub), static_cast<unsigned>(p.batch)),
                       dim3(kThreads), 0, stream, a.B, a.C, a.g, a.cp, a.bt, p.seqlen, p.nsub);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (in.flags & kFwdOnly) return launch_dirs<1>(a, p.batch, stream, stage);
  if (in.flags & kRevOnly) return launch_dirs<2>(a, p.batch, stream, stage);
  return launch_dirs<3>(a, p.batch, stream, stage);
}

}  // namespace ssd
}  // namespace bimamba
