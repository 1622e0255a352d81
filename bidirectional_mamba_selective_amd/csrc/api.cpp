// C ABI of the bidirectional selective-scan library (declared in include/bimamba.h).
// Every argument is validated here, before any HIP call.
#include "../../include/bimamba.h"

#include <stdint.h>

#include <algorithm>

#include "launch.h"
#include "plan.h"

namespace {

using bimamba::Plan;

constexpr uint32_t kKnownFlags = BIMAMBA_FLAG_NO_GATE | BIMAMBA_FLAG_FWD_ONLY | BIMAMBA_FLAG_REV_ONLY;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shape check shared by both entry points.
int check_shape(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype) {
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_state <= 0) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (io_dtype != BIMAMBA_F32 && io_dtype != BIMAMBA_BF16) return BIMAMBA_ERR_UNSUPPORTED;
  if (d_inner % bimamba::kLanes != 0 || d_state > 16) return BIMAMBA_ERR_UNSUPPORTED;
  // grid and index limits of the kernels: int token/channel indices, 16-bit grid y/z
  if (seqlen > INT32_MAX / 2 || d_inner > INT32_MAX / 2 || batch > 65535) return BIMAMBA_ERR_UNSUPPORTED;
  if (static_cast<double>(batch) * seqlen * d_inner > 9.0e15) return BIMAMBA_ERR_UNSUPPORTED;
  // The chunked kernels address a tile's rows, a tile boundary's states and the carries through buffer
  // resources with 32-bit byte offsets and a range of at most 2^31 - 1 bytes: a tile of kSub token rows
  // of d_inner elements, and d_state rows of d_inner fp32 states (plus one 256-byte row of slack), must fit.
  const int64_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  if (bimamba::kSub * d_inner * es > INT32_MAX || d_state * d_inner * 4 + 256 > INT32_MAX)
    return BIMAMBA_ERR_UNSUPPORTED;
  return BIMAMBA_OK;
}

// Whether r overlaps any input of a scan call (x, dt, z [batch, seqlen, d_inner]; B, C [batch, seqlen, d_state];
// A [d_inner, d_state]; D, dt_bias [d_inner]); z, D and dt_bias may be NULL.
bool hits_scan_inputs(Range r, const void* x, const void* dt, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* dt_bias, int64_t batch, int64_t seqlen,
                      int64_t d_inner, int64_t d_state, int io_dtype) {
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  const size_t act = static_cast<size_t>(batch) * seqlen * d_inner * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * d_state * es;
  return overlap(r, range_of(x, act)) || overlap(r, range_of(dt, act)) || overlap(r, range_of(B, bc)) ||
         overlap(r, range_of(C, bc)) || (z && overlap(r, range_of(z, act))) ||
         overlap(r, range_of(A, static_cast<size_t>(d_inner) * d_state * 4)) ||
         (D && overlap(r, range_of(D, static_cast<size_t>(d_inner) * 4))) ||
         (dt_bias && overlap(r, range_of(dt_bias, static_cast<size_t>(d_inner) * 4)));
}

// Pointer checks shared by both entry points; sizes in elements.
int check_tensors(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* dt_bias, void* out, int64_t batch, int64_t seqlen, int64_t d_inner,
                  int64_t d_state, int io_dtype, uint32_t flags) {
  if (flags & ~kKnownFlags) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if ((flags & BIMAMBA_FLAG_FWD_ONLY) && (flags & BIMAMBA_FLAG_REV_ONLY)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!x || !dt || !A || !B || !C || !out) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!z && !(flags & BIMAMBA_FLAG_NO_GATE)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  if (!aligned(x, 16) || !aligned(dt, 16) || !aligned(out, 16) || (z && !aligned(z, 16))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!aligned(B, es) || !aligned(C, es)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!aligned(A, 16) || (D && !aligned(D, 16)) || (dt_bias && !aligned(dt_bias, 16))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const Range o = range_of(out, static_cast<size_t>(batch) * seqlen * d_inner * es);
  if (hits_scan_inputs(o, x, dt, A, B, C, D, z, dt_bias, batch, seqlen, d_inner, d_state, io_dtype))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  return BIMAMBA_OK;
}

int check_workspace(const Plan& p, void* workspace, size_t workspace_bytes, void* out, size_t out_bytes) {
  if (workspace_bytes < p.total) return BIMAMBA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 256)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (overlap(range_of(workspace, p.total), range_of(out, out_bytes))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  return BIMAMBA_OK;
}

int map_hip(hipError_t e) { return e == hipSuccess ? BIMAMBA_OK : BIMAMBA_ERR_HIP; }

}  // namespace

extern "C" {

int bimamba_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* bimamba_status_string(int status) {
  switch (status) {
    case BIMAMBA_OK: return "ok";
    case BIMAMBA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BIMAMBA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BIMAMBA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case BIMAMBA_ERR_HIP: return "HIP launch error";
    case BIMAMBA_ERR_SCRATCH_TOO_SMALL: return "problem too large for the library's 256 MiB scratch buffer";
    default: return "unknown status";
  }
}

size_t bimamba_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  // the size does not depend on the I/O dtype; bf16 admits the larger shapes
  if (check_shape(batch, seqlen, d_inner, d_state, BIMAMBA_BF16) != BIMAMBA_OK) return 0;
  return bimamba::make_plan(batch, seqlen, d_inner, d_state).total;
}

static int scan_fwd_impl(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* dt_bias, void* out, int64_t batch,
                         int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, uint32_t flags,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < -1 || stage > 2) return BIMAMBA_ERR_INVALID_ARGUMENT;
  int s = check_shape(batch, seqlen, d_inner, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  s = check_tensors(x, dt, A, B, C, D, z, dt_bias, out, batch, seqlen, d_inner, d_state, io_dtype, flags);
  if (s != BIMAMBA_OK) return s;
  const Plan p = bimamba::make_plan(batch, seqlen, d_inner, d_state);
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  s = check_workspace(p, workspace, workspace_bytes, out, static_cast<size_t>(batch) * seqlen * d_inner * es);
  if (s != BIMAMBA_OK) return s;
  // the kernels write the workspace while others still read the inputs
  if (hits_scan_inputs(range_of(workspace, p.total), x, dt, A, B, C, D, z, dt_bias, batch, seqlen, d_inner, d_state,
                       io_dtype))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  bimamba::ScanArgs a{x, dt, A, B, C, D, z, dt_bias, out, nullptr, nullptr, io_dtype, flags};
  return map_hip(bimamba::launch_chunked(a, p, workspace, stream, stage));
}

int bimamba_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                     const void* z, const float* dt_bias, void* out, int64_t batch, int64_t seqlen, int64_t d_inner,
                     int64_t d_state, int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return scan_fwd_impl(-1, x, dt, A, B, C, D, z, dt_bias, out, batch, seqlen, d_inner, d_state, io_dtype, flags,
                       workspace, workspace_bytes, stream);
}

int bimamba_scan_fwd_stage(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, void* out, int64_t batch,
                           int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return scan_fwd_impl(stage, x, dt, A, B, C, D, z, dt_bias, out, batch, seqlen, d_inner, d_state, io_dtype, flags,
                       workspace, workspace_bytes, stream);
}

int bimamba_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* dt_bias, void* out, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, uint32_t flags,
                             hipStream_t stream) {
  int s = check_shape(batch, seqlen, d_inner, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  s = check_tensors(x, dt, A, B, C, D, z, dt_bias, out, batch, seqlen, d_inner, d_state, io_dtype, flags);
  if (s != BIMAMBA_OK) return s;
  const Plan p = bimamba::make_plan(batch, seqlen, d_inner, d_state);
  if (p.total > bimamba::kScratchBytes) return BIMAMBA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (bimamba::scratch_address(&ws) != hipSuccess) return BIMAMBA_ERR_HIP;
  // out must not overlap the scratch array (the library's own memory, so only a caller that passed a
  // pointer into it could make them overlap)
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  if (overlap(range_of(ws, bimamba::kScratchBytes),
              range_of(out, static_cast<size_t>(batch) * seqlen * d_inner * es)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  bimamba::ScanArgs a{x, dt, A, B, C, D, z, dt_bias, out, nullptr, nullptr, io_dtype, flags};
  return map_hip(bimamba::launch_chunked(a, p, ws, stream));
}

int bimamba_scan_fwd_untied(const void* x_f, const void* dt_f, const float* A_f, const void* B_f, const void* C_f,
                            const float* D_f, const void* z_f, const float* dt_bias_f, void* out_f, const void* x_r,
                            const void* dt_r, const float* A_r, const void* B_r, const void* C_r, const float* D_r,
                            const void* z_r, const float* dt_bias_r, void* out_r, int64_t batch, int64_t seqlen,
                            int64_t d_inner, int64_t d_state, int io_dtype, uint32_t flags, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  int s = check_shape(batch, seqlen, d_inner, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  if (flags & ~static_cast<uint32_t>(BIMAMBA_FLAG_NO_GATE)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  s = check_tensors(x_f, dt_f, A_f, B_f, C_f, D_f, z_f, dt_bias_f, out_f, batch, seqlen, d_inner, d_state, io_dtype,
                    flags);
  if (s != BIMAMBA_OK) return s;
  s = check_tensors(x_r, dt_r, A_r, B_r, C_r, D_r, z_r, dt_bias_r, out_r, batch, seqlen, d_inner, d_state, io_dtype,
                    flags);
  if (s != BIMAMBA_OK) return s;
  // the reverse pass runs after the forward one: out_f must not overlap anything the reverse pass
  // reads or writes, nor out_r anything of the forward pass
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  const size_t act = static_cast<size_t>(batch) * seqlen * d_inner * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * d_state * es;
  const size_t par = static_cast<size_t>(d_inner) * d_state * 4, vec = static_cast<size_t>(d_inner) * 4;
  auto hits = [&](const void* out, const void* x, const void* dt, const float* A, const void* B, const void* C,
                  const float* D, const void* z, const float* bias) {
    const Range o = range_of(out, act);
    return overlap(o, range_of(x, act)) || overlap(o, range_of(dt, act)) || overlap(o, range_of(B, bc)) ||
           overlap(o, range_of(C, bc)) || (z && overlap(o, range_of(z, act))) || overlap(o, range_of(A, par)) ||
           (D && overlap(o, range_of(D, vec))) || (bias && overlap(o, range_of(bias, vec)));
  };
  if (hits(out_f, x_r, dt_r, A_r, B_r, C_r, D_r, z_r, dt_bias_r) ||
      hits(out_r, x_f, dt_f, A_f, B_f, C_f, D_f, z_f, dt_bias_f) || overlap(range_of(out_f, act), range_of(out_r, act)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  const Plan p = bimamba::make_plan(batch, seqlen, d_inner, d_state);
  s = check_workspace(p, workspace, workspace_bytes, out_f, act);
  if (s != BIMAMBA_OK) return s;
  const Range wr = range_of(workspace, p.total);
  if (overlap(wr, range_of(out_r, act)) ||
      hits_scan_inputs(wr, x_f, dt_f, A_f, B_f, C_f, D_f, z_f, dt_bias_f, batch, seqlen, d_inner, d_state, io_dtype) ||
      hits_scan_inputs(wr, x_r, dt_r, A_r, B_r, C_r, D_r, z_r, dt_bias_r, batch, seqlen, d_inner, d_state, io_dtype))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  // two one-direction passes in stream order, sharing the workspace
  const bimamba::ScanArgs af{x_f, dt_f, A_f, B_f, C_f, D_f, z_f, dt_bias_f, out_f, nullptr, nullptr, io_dtype,
                             flags | BIMAMBA_FLAG_FWD_ONLY};
  s = map_hip(bimamba::launch_chunked(af, p, workspace, stream));
  if (s != BIMAMBA_OK) return s;
  const bimamba::ScanArgs ar{x_r, dt_r, A_r, B_r, C_r, D_r, z_r, dt_bias_r, out_r, nullptr, nullptr, io_dtype,
                             flags | BIMAMBA_FLAG_REV_ONLY};
  return map_hip(bimamba::launch_chunked(ar, p, workspace, stream));
}

size_t bimamba_scan_block_workspace_bytes(int64_t batch, int64_t block_len, int64_t d_inner, int64_t d_state) {
  if (check_shape(batch, block_len, d_inner, d_state, BIMAMBA_BF16) != BIMAMBA_OK) return 0;
  if (block_len <= bimamba::kBlockFusedMax) return 0;  // single-kernel path
  return bimamba::make_plan(batch, block_len, d_inner, d_state).total;
}

int bimamba_scan_block(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                       const void* z, const float* dt_bias, const float* h_in, float* h_out, void* out,
                       int64_t batch, int64_t block_len, int64_t d_inner, int64_t d_state, int io_dtype,
                       uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int s = check_shape(batch, block_len, d_inner, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  s = check_tensors(x, dt, A, B, C, D, z, dt_bias, out, batch, block_len, d_inner, d_state, io_dtype, flags);
  if (s != BIMAMBA_OK) return s;
  const size_t st_bytes = static_cast<size_t>(batch) * d_inner * d_state * sizeof(float);
  if ((h_in && !aligned(h_in, 16)) || (h_out && !aligned(h_out, 16))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_in && h_out && h_in != h_out && overlap(range_of(h_in, st_bytes), range_of(h_out, st_bytes)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  const size_t out_bytes = static_cast<size_t>(batch) * block_len * d_inner * es;
  if (h_out && overlap(range_of(h_out, st_bytes), range_of(out, out_bytes))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_in && overlap(range_of(h_in, st_bytes), range_of(out, out_bytes))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_out) {
    // the new cache is written while other workgroups still read the block's inputs
    const Range ho = range_of(h_out, st_bytes);
    const size_t act = static_cast<size_t>(batch) * block_len * d_inner * es;
    const size_t bc = static_cast<size_t>(batch) * block_len * d_state * es;
    if (overlap(ho, range_of(x, act)) || overlap(ho, range_of(dt, act)) || (z && overlap(ho, range_of(z, act))) ||
        overlap(ho, range_of(B, bc)) || overlap(ho, range_of(C, bc)) ||
        overlap(ho, range_of(A, static_cast<size_t>(d_inner) * d_state * 4)) ||
        (D && overlap(ho, range_of(D, static_cast<size_t>(d_inner) * 4))) ||
        (dt_bias && overlap(ho, range_of(dt_bias, static_cast<size_t>(d_inner) * 4))))
      return BIMAMBA_ERR_INVALID_ARGUMENT;
  }
  bimamba::ScanArgs a{x, dt, A, B, C, D, z, dt_bias, out, h_in, h_out, io_dtype, flags};
  if (block_len <= bimamba::kBlockFusedMax) {
    // single-kernel path: the workspace is not used (it may be NULL)
    return map_hip(bimamba::launch_block_fused(a, batch, block_len, d_inner, d_state, stream));
  }
  const Plan p = bimamba::make_plan(batch, block_len, d_inner, d_state);
  s = check_workspace(p, workspace, workspace_bytes, out, out_bytes);
  if (s != BIMAMBA_OK) return s;
  // the staging and summary kernels write the workspace before the carry kernel reads h_in
  const Range wr = range_of(workspace, p.total);
  if ((h_out && overlap(range_of(h_out, st_bytes), wr)) || (h_in && overlap(range_of(h_in, st_bytes), wr)) ||
      hits_scan_inputs(wr, x, dt, A, B, C, D, z, dt_bias, batch, block_len, d_inner, d_state, io_dtype))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  return map_hip(bimamba::launch_chunked(a, p, workspace, stream));
}

// ---- Mamba-2 (SSD) heads ----

static int ssd_check_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                           int io_dtype) {
  namespace ssd = bimamba::ssd;
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || d_state <= 0) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (io_dtype != BIMAMBA_F32 && io_dtype != BIMAMBA_BF16) return BIMAMBA_ERR_UNSUPPORTED;
  if (io_dtype != BIMAMBA_BF16 || headdim != ssd::kHeadDim || d_state != ssd::kState) return BIMAMBA_ERR_UNSUPPORTED;
  // grid limits: (sub-chunks, batch) for the tiling kernel, one workgroup per (batch, chunk, head) otherwise
  // a run's output rows (64 tokens of nheads * headdim bf16 channels) are stored through one buffer
  // resource whose range is at most 2^31 - 1 bytes
  if (batch > 65535 || nheads > (1 << 18) || seqlen > INT32_MAX / 2) return BIMAMBA_ERR_UNSUPPORTED;
  const bimamba::ssd::SsdPlan p = bimamba::ssd::make_ssd_plan(batch, seqlen, nheads);
  if (static_cast<double>(batch) * p.nchunk * nheads > 2.0e9 ||
      static_cast<double>(batch) * nheads * ssd::kStateFloats > 2.0e9)
    return BIMAMBA_ERR_UNSUPPORTED;
  return BIMAMBA_OK;
}

// ssd_impl's stage value for the single-kernel block step (blocks of at most one run)
constexpr int kSsdBlockFused = -2;

static int ssd_impl(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* dt_bias, const float* h_in, float* h_out, void* out,
                    int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state, int io_dtype,
                    uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if ((stage < -1 || stage > 3) && stage != kSsdBlockFused) return BIMAMBA_ERR_INVALID_ARGUMENT;
  int s = ssd_check_shape(batch, seqlen, nheads, headdim, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  if (flags & ~kKnownFlags) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if ((flags & BIMAMBA_FLAG_FWD_ONLY) && (flags & BIMAMBA_FLAG_REV_ONLY)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!x || !dt || !A || !B || !C || !out) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!z && !(flags & BIMAMBA_FLAG_NO_GATE)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(B, 16) || !aligned(C, 16) || (z && !aligned(z, 16)) ||
      !aligned(dt, 2) || !aligned(A, 4) || (D && !aligned(D, 4)) || (dt_bias && !aligned(dt_bias, 4)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  const size_t act = static_cast<size_t>(batch) * seqlen * nheads * headdim * 2;
  const size_t dtb = static_cast<size_t>(batch) * seqlen * nheads * 2;
  const size_t bc = static_cast<size_t>(batch) * seqlen * d_state * 2;
  const size_t par = static_cast<size_t>(nheads) * 4;
  const Range o = range_of(out, act);
  if (overlap(o, range_of(x, act)) || overlap(o, range_of(dt, dtb)) || overlap(o, range_of(B, bc)) ||
      overlap(o, range_of(C, bc)) || (z && overlap(o, range_of(z, act))) || overlap(o, range_of(A, par)) ||
      (D && overlap(o, range_of(D, par))) || (dt_bias && overlap(o, range_of(dt_bias, par))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  // block decoding: the cached forward state in and out ([batch, nheads, headdim, d_state] fp32)
  const size_t stb = static_cast<size_t>(batch) * nheads * headdim * d_state * 4;
  if ((h_in && !aligned(h_in, 4)) || (h_out && !aligned(h_out, 4))) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_out && (flags & BIMAMBA_FLAG_REV_ONLY)) return BIMAMBA_ERR_INVALID_ARGUMENT;  // no forward state computed
  if (h_in && h_out && h_in != h_out && overlap(range_of(h_in, stb), range_of(h_out, stb)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_in && overlap(range_of(h_in, stb), o)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (h_out) {
    const Range ho = range_of(h_out, stb);
    if (overlap(ho, o) || overlap(ho, range_of(x, act)) || overlap(ho, range_of(dt, dtb)) ||
        overlap(ho, range_of(B, bc)) || overlap(ho, range_of(C, bc)) || (z && overlap(ho, range_of(z, act))) ||
        overlap(ho, range_of(A, par)) || (D && overlap(ho, range_of(D, par))) ||
        (dt_bias && overlap(ho, range_of(dt_bias, par))))
      return BIMAMBA_ERR_INVALID_ARGUMENT;
  }
  const bimamba::ssd::SsdArgs a{x, dt, A, B, C, D, z, dt_bias, out, flags, h_in, h_out};
  if (stage == kSsdBlockFused) {
    // a block of at most one run: one kernel, no workspace
    return map_hip(bimamba::ssd::launch_ssd_block(a, batch, seqlen, nheads, stream));
  }
  const bimamba::ssd::SsdPlan p = bimamba::ssd::make_ssd_plan(batch, seqlen, nheads);
  if (workspace_bytes < p.total) return BIMAMBA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 256)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const Range wr = range_of(workspace, p.total);
  if (overlap(wr, o) || (h_in && overlap(wr, range_of(h_in, stb))) || (h_out && overlap(wr, range_of(h_out, stb))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  // the tiling kernel and the sweeps write the workspace while others still read the inputs
  if (overlap(wr, range_of(x, act)) || overlap(wr, range_of(dt, dtb)) || overlap(wr, range_of(B, bc)) ||
      overlap(wr, range_of(C, bc)) || (z && overlap(wr, range_of(z, act))) || overlap(wr, range_of(A, par)) ||
      (D && overlap(wr, range_of(D, par))) || (dt_bias && overlap(wr, range_of(dt_bias, par))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  return map_hip(bimamba::ssd::launch_ssd(a, p, workspace, stream, stage));
}

size_t bimamba_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t d_state) {
  if (ssd_check_shape(batch, seqlen, nheads, headdim, d_state, BIMAMBA_BF16) != BIMAMBA_OK) return 0;
  return bimamba::ssd::make_ssd_plan(batch, seqlen, nheads).total;
}

int bimamba_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                    const void* z, const float* dt_bias, void* out, int64_t batch, int64_t seqlen, int64_t nheads,
                    int64_t headdim, int64_t d_state, int io_dtype, uint32_t flags, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return ssd_impl(-1, x, dt, A, B, C, D, z, dt_bias, nullptr, nullptr, out, batch, seqlen, nheads, headdim, d_state,
                  io_dtype, flags, workspace, workspace_bytes, stream);
}

int bimamba_ssd_fwd_stage(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* dt_bias, void* out, int64_t batch,
                          int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state, int io_dtype,
                          uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 0) return BIMAMBA_ERR_INVALID_ARGUMENT;
  return ssd_impl(stage, x, dt, A, B, C, D, z, dt_bias, nullptr, nullptr, out, batch, seqlen, nheads, headdim,
                  d_state, io_dtype, flags, workspace, workspace_bytes, stream);
}

size_t bimamba_ssd_block_workspace_bytes(int64_t batch, int64_t block_len, int64_t nheads, int64_t headdim,
                                         int64_t d_state) {
  if (block_len <= bimamba::ssd::kQ) return 0;  // single-kernel path
  return bimamba_ssd_fwd_workspace_bytes(batch, block_len, nheads, headdim, d_state);
}

int bimamba_ssd_block(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                      const void* z, const float* dt_bias, const float* h_in, float* h_out, void* out,
                      int64_t batch, int64_t block_len, int64_t nheads, int64_t headdim, int64_t d_state,
                      int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ssd_impl(block_len <= bimamba::ssd::kQ ? kSsdBlockFused : -1, x, dt, A, B, C, D, z, dt_bias, h_in, h_out,
                  out, batch, block_len, nheads, headdim, d_state, io_dtype, flags, workspace, workspace_bytes, stream);
}

int bimamba_ssd_conv_untied(const void* xbc_f, const float* cw_f, const float* cb_f, const void* dt_f,
                            const float* A_f, const float* D_f, const void* z_f, const float* dt_bias_f, void* out_f,
                            const void* xbc_r, const float* cw_r, const float* cb_r, const void* dt_r,
                            const float* A_r, const float* D_r, const void* z_r, const float* dt_bias_r, void* out_r,
                            int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t d_conv, int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  int s = ssd_check_shape(batch, seqlen, nheads, headdim, d_state, io_dtype);
  if (s != BIMAMBA_OK) return s;
  if (d_conv != 4) return d_conv <= 0 ? BIMAMBA_ERR_INVALID_ARGUMENT : BIMAMBA_ERR_UNSUPPORTED;
  if (flags & ~static_cast<uint32_t>(BIMAMBA_FLAG_NO_GATE)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!out_f && !out_r) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const bool gate = !(flags & BIMAMBA_FLAG_NO_GATE);
  const int64_t xs = nheads * headdim + 2 * d_state;  // stream channels: x, then B, then C
  // with the convolution, a head's window rows are loaded through a buffer resource over one batch
  // element's stream with 32-bit byte offsets
  if ((cw_f || cw_r) && seqlen * xs * 2 + 256 > INT32_MAX) return BIMAMBA_ERR_UNSUPPORTED;
  const size_t act_x = static_cast<size_t>(batch) * seqlen * xs * 2;
  const size_t act_o = static_cast<size_t>(batch) * seqlen * nheads * headdim * 2;
  const size_t dtb = static_cast<size_t>(batch) * seqlen * nheads * 2;
  const size_t par = static_cast<size_t>(nheads) * 4;
  const size_t cwb = static_cast<size_t>(xs) * 4 * 4, cbb = static_cast<size_t>(xs) * 4;
  struct Set {
    const void* xbc; const float* cw; const float* cb; const void* dt; const float* A; const float* D;
    const void* z; const float* bias; void* out;
  };
  const Set sets[2] = {{xbc_f, cw_f, cb_f, dt_f, A_f, D_f, z_f, dt_bias_f, out_f},
                       {xbc_r, cw_r, cb_r, dt_r, A_r, D_r, z_r, dt_bias_r, out_r}};
  for (const Set& t : sets) {
    if (!t.out) continue;
    if (!t.xbc || !t.dt || !t.A || (gate && !t.z)) return BIMAMBA_ERR_INVALID_ARGUMENT;
    if (!aligned(t.xbc, 16) || !aligned(t.out, 16) || (t.z && !aligned(t.z, 16)) || !aligned(t.dt, 2) ||
        !aligned(t.A, 4) || (t.D && !aligned(t.D, 4)) || (t.bias && !aligned(t.bias, 4)) ||
        (t.cw && !aligned(t.cw, 4)) || (t.cb && !aligned(t.cb, 4)))
      return BIMAMBA_ERR_INVALID_ARGUMENT;
  }
  // an output may not overlap anything either pass reads or writes
  auto clash = [&](Range o) {
    for (const Set& t : sets) {
      if (!t.out) continue;
      if (overlap(o, range_of(t.xbc, act_x)) || overlap(o, range_of(t.dt, dtb)) || overlap(o, range_of(t.A, par)) ||
          (t.D && overlap(o, range_of(t.D, par))) || (t.bias && overlap(o, range_of(t.bias, par))) ||
          (t.z && overlap(o, range_of(t.z, act_o))) || (t.cw && overlap(o, range_of(t.cw, cwb))) ||
          (t.cb && overlap(o, range_of(t.cb, cbb))))
        return true;
    }
    return false;
  };
  if ((out_f && clash(range_of(out_f, act_o))) || (out_r && clash(range_of(out_r, act_o))) ||
      (out_f && out_r && overlap(range_of(out_f, act_o), range_of(out_r, act_o))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  const bimamba::ssd::SsdPlan p = bimamba::ssd::make_ssd_plan(batch, seqlen, nheads);
  if (workspace_bytes < p.total) return BIMAMBA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 256)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const Range wr = range_of(workspace, p.total);
  if ((out_f && overlap(wr, range_of(out_f, act_o))) || (out_r && overlap(wr, range_of(out_r, act_o))) ||
      clash(wr))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  // the forward layer, then the reverse layer, in stream order, sharing the workspace
  for (int d = 0; d < 2; ++d) {
    const Set& t = sets[d];
    if (!t.out) continue;
    const bimamba::ssd::SsdArgs a{t.xbc, t.dt, t.A, nullptr, nullptr, t.D, t.z, t.bias, t.out, flags, nullptr, nullptr};
    s = map_hip(bimamba::ssd::launch_ssd_one_dir(a, t.cw, t.cb, xs, p, workspace, d + 1, stream));
    if (s != BIMAMBA_OK) return s;
  }
  return BIMAMBA_OK;
}

// ---- Short causal / anti-causal convolution ----

static int conv_impl(const void* u, const float* w_f, const float* b_f, const float* w_r, const float* b_r,
                     const void* cache_in, void* cache_out, void* out_f, void* out_r, int64_t batch, int64_t L,
                     int64_t C, int64_t d_conv, int io_dtype, uint32_t flags, hipStream_t stream, bool block) {
  if (batch <= 0 || L <= 0 || C <= 0 || d_conv <= 0) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (io_dtype != BIMAMBA_F32 && io_dtype != BIMAMBA_BF16) return BIMAMBA_ERR_UNSUPPORTED;
  if (d_conv != 4 || C % 4 != 0 || C > (int64_t{1} << 22)) return BIMAMBA_ERR_UNSUPPORTED;  // a tile's rows fit a buffer
  if (batch > 65535 || L > INT32_MAX / 2 || static_cast<double>((L + 63) / 64) * ((C / 4 + 255) / 256) > 2.0e9)
    return BIMAMBA_ERR_UNSUPPORTED;
  if (flags & ~static_cast<uint32_t>(BIMAMBA_FLAG_NO_SILU)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!u || (!out_f && !out_r)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if ((out_f && !w_f) || (out_r && !w_r)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (!block && (cache_in || cache_out)) return BIMAMBA_ERR_INVALID_ARGUMENT;
  const size_t es = io_dtype == BIMAMBA_BF16 ? 2 : 4;
  const uintptr_t va = 4 * es;
  if (!aligned(u, va) || (out_f && !aligned(out_f, va)) || (out_r && !aligned(out_r, va)) ||
      (cache_in && !aligned(cache_in, va)) || (cache_out && !aligned(cache_out, va)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  if ((w_f && !aligned(w_f, 4)) || (w_r && !aligned(w_r, 4)) || (b_f && !aligned(b_f, 4)) ||
      (b_r && !aligned(b_r, 4)))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  const size_t act = static_cast<size_t>(batch) * L * C * es;
  const size_t cb = static_cast<size_t>(batch) * 3 * C * es;
  const size_t wb = static_cast<size_t>(C) * d_conv * 4, bb = static_cast<size_t>(C) * 4;
  // everything an output may not touch
  auto clash = [&](Range o) {
    return overlap(o, range_of(u, act)) || (w_f && overlap(o, range_of(w_f, wb))) ||
           (w_r && overlap(o, range_of(w_r, wb))) || (b_f && overlap(o, range_of(b_f, bb))) ||
           (b_r && overlap(o, range_of(b_r, bb))) || (cache_in && overlap(o, range_of(cache_in, cb)));
  };
  if (out_f && (clash(range_of(out_f, act)) || (out_r && overlap(range_of(out_f, act), range_of(out_r, act))) ||
                (cache_out && overlap(range_of(out_f, act), range_of(cache_out, cb)))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (out_r && (clash(range_of(out_r, act)) || (cache_out && overlap(range_of(out_r, act), range_of(cache_out, cb)))))
    return BIMAMBA_ERR_INVALID_ARGUMENT;
  if (cache_out) {
    const Range co = range_of(cache_out, cb);
    const bool in_place = cache_in == cache_out;
    if (overlap(co, range_of(u, act)) || (w_f && overlap(co, range_of(w_f, wb))) ||
        (w_r && overlap(co, range_of(w_r, wb))) || (b_f && overlap(co, range_of(b_f, bb))) ||
        (b_r && overlap(co, range_of(b_r, bb))) || (cache_in && !in_place && overlap(co, range_of(cache_in, cb))))
      return BIMAMBA_ERR_INVALID_ARGUMENT;
  }
  const bimamba::conv::ConvArgs a{u, w_f, b_f, w_r, b_r, cache_in, cache_out, out_f, out_r,
                                  (flags & BIMAMBA_FLAG_NO_SILU) ? 0 : 1};
  return map_hip(bimamba::conv::launch_conv(a, batch, L, C, io_dtype, stream));
}

int bimamba_conv1d_bidir(const void* u, const float* w_f, const float* b_f, const float* w_r, const float* b_r,
                         void* out_f, void* out_r, int64_t batch, int64_t seqlen, int64_t channels, int64_t d_conv,
                         int io_dtype, uint32_t flags, hipStream_t stream) {
  return conv_impl(u, w_f, b_f, w_r, b_r, nullptr, nullptr, out_f, out_r, batch, seqlen, channels, d_conv, io_dtype,
                   flags, stream, false);
}

int bimamba_conv1d_block(const void* u, const float* w_f, const float* b_f, const float* w_r, const float* b_r,
                         const void* cache_in, void* cache_out, void* out_f, void* out_r, int64_t batch,
                         int64_t block_len, int64_t channels, int64_t d_conv, int io_dtype, uint32_t flags,
                         hipStream_t stream) {
  return conv_impl(u, w_f, b_f, w_r, b_r, cache_in, cache_out, out_f, out_r, batch, block_len, channels, d_conv,
                   io_dtype, flags, stream, true);
}

}  // extern "C"
