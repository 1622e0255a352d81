// Host-side decomposition of the Mamba-2 (SSD) scan into runs and chunks, and
// the layout of its workspace.  Pure host code: no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace bimamba {
namespace ssd {

constexpr int64_t kHeadDim = 32;   // channels per head
constexpr int64_t kState = 128;    // state size
constexpr int64_t kQ = 64;         // tokens per run (the matrix-core tile height)
constexpr int64_t kStateFloats = kHeadDim * kState;
// Workgroups the chunking aims to give each walking pass (two per CU resident).
constexpr int64_t kTargetGroups = 2048;
// Shortest chunk, in runs: below it the chunk states cost more traffic than the activations.
constexpr int64_t kMinRuns = 4;

struct SsdPlan {
  int64_t batch, seqlen, nheads;
  int64_t nsub;    // runs per sequence
  int64_t rpc;     // runs per chunk
  int64_t nchunk;  // chunks per sequence
  // workspace offsets in bytes (each 256-byte aligned)
  size_t off_g, off_cp, off_bt, off_s, off_p, off_tau, total;
};

inline SsdPlan make_ssd_plan(int64_t batch, int64_t seqlen, int64_t nheads) {
  SsdPlan p{};
  p.batch = batch;
  p.seqlen = seqlen;
  p.nheads = nheads;
  p.nsub = (seqlen + kQ - 1) / kQ;
  int64_t want = kTargetGroups / (batch * nheads);
  if (want < 1) want = 1;
  int64_t rpc = (p.nsub + want - 1) / want;
  if (rpc < kMinRuns) rpc = kMinRuns;
  if (rpc > p.nsub) rpc = p.nsub;
  p.rpc = rpc;
  p.nchunk = (p.nsub + rpc - 1) / rpc;
  const size_t tile = static_cast<size_t>(batch) * p.nsub * kQ * kState * 2;  // bf16 [Q][N] per run
  const size_t gt = static_cast<size_t>(batch) * p.nsub * kQ * kQ * 4;       // fp32 [Q][Q] per run
  const size_t items = static_cast<size_t>(batch) * p.nchunk * nheads;
  size_t off = 0;
  p.off_g = off;   off = align256(off + gt);
  p.off_cp = off;  off = align256(off + tile);
  p.off_bt = off;  off = align256(off + tile);
  p.off_s = off;   off = align256(off + items * 2 * kStateFloats * sizeof(float));
  p.off_p = off;   off = align256(off + items * sizeof(float));
  p.off_tau = off; off = align256(off + items * static_cast<size_t>(rpc) * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace ssd
}  // namespace bimamba
