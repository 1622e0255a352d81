// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"
#include "ssd_plan.h"

namespace bimamba {

enum : uint32_t { kNoGate = 1u, kFwdOnly = 2u, kRevOnly = 4u };

struct ScanArgs {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* out;
  const float* h_in;  // forward state entering the sequence (NULL = zeros)
  float* h_out;       // forward state after the last token (NULL = not written)
  int io_dtype;       // 0 = fp32, 1 = bf16
  uint32_t flags;
};

// Three-kernel chunked scan (summary -> carry -> output) for any length.
// stage < 0 launches all three; 0, 1, 2 launch one of them.
hipError_t launch_chunked(const ScanArgs& a, const Plan& p, void* workspace, hipStream_t stream, int stage = -1);

// Size of the library's fixed device scratch array (csrc/scratch.hip), which holds the workspace of
// the allocation-free entry point.
constexpr size_t kScratchBytes = size_t{256} << 20;

// Address of the scratch array on the current device (looked up once per device).
hipError_t scratch_address(void** out);

// Single-kernel block step for block_len <= kBlockFusedMax: one workgroup per
// (16 channels, batch element), one lane per (channel, state) recurrence; no workspace.
hipError_t launch_block_fused(const ScanArgs& a, int64_t batch, int64_t block_len, int64_t d_inner,
                              int64_t d_state, hipStream_t stream);

namespace conv {

// Short causal / anti-causal depthwise convolution (width 4) with optional SiLU.
struct ConvArgs {
  const void* u;
  const float* w_f;
  const float* b_f;
  const float* w_r;
  const float* b_r;
  const void* cache_in;  // block decoding: the 3 tokens before the block (null = zeros)
  void* cache_out;       // block decoding: receives the last 3 tokens (null = not written)
  void* out_f;           // null = forward direction not computed
  void* out_r;           // null = reverse direction not computed
  int act;
};

hipError_t launch_conv(const ConvArgs& a, int64_t batch, int64_t L, int64_t C, int io_dtype, hipStream_t stream);

}  // namespace conv

namespace ssd {

// Mamba-2 (SSD) scan: bf16 x, dt, B, C, z, out; fp32 A, D, dt_bias per head.
struct SsdArgs {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* out;
  uint32_t flags;
  const float* h_in;  // block decoding: forward state entering the sequence (null = zeros)
  float* h_out;       // block decoding: receives the forward state after it (null = not written)
};

// Staged chunked scan: stage 0 tiles B and C, 1 chunk summaries, 2 carry,
// 3 output; stage < 0 launches all four.  h_in / h_out enter and leave
// through the carry stage.
hipError_t launch_ssd(const SsdArgs& a, const SsdPlan& p, void* workspace, hipStream_t stream, int stage = -1);

// One direction of a Mamba-2 layer (dir 1 forward, 2 reverse) on a projection stream of xs elements per token
// holding x, B and C as channels [0, H*P), [H*P, H*P+N), [H*P+N, H*P+2N) (in.x is the stream; in.B, in.C,
// in.h_in and in.h_out are not used), with the short convolution of taps cw [xs, 4] and bias cb applied to
// the stream first when cw is not null: causal for dir 1, anti-causal for dir 2.
hipError_t launch_ssd_one_dir(const SsdArgs& in, const float* cw, const float* cb, int64_t xs, const SsdPlan& p,
                              void* workspace, int dir, hipStream_t stream);

// One block-cache decoding step of at most kQ tokens in a single kernel (no workspace).
hipError_t launch_ssd_block(const SsdArgs& a, int64_t batch, int64_t block_len, int64_t nheads, hipStream_t stream);

}  // namespace ssd

}  // namespace bimamba
