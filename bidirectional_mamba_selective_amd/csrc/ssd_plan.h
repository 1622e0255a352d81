// Host-side decomposition of the Mamba-2 (SSD) scan into sub-chunks, segments
// and chunks, and the layout of its workspace.  Pure host code: no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace bimamba {
namespace ssd {

constexpr int64_t kHeadDim = 32;   // channels per head
constexpr int64_t kState = 128;    // state size
constexpr int64_t kQ = 64;         // tokens per sub-chunk (one matrix-core tile row block)
constexpr int64_t kSeg = 8;        // sub-chunks per segment (the output pass stashes a segment in LDS)
constexpr int64_t kStateFloats = kHeadDim * kState;
// Workgroups the chunking aims to give the summary and output passes.
constexpr int64_t kTargetGroups = 2048;

struct SsdPlan {
  int64_t batch, seqlen, nheads;
  int64_t nsub;   // sub-chunks per sequence
  int64_t nseg;   // segments per sequence
  int64_t spc;    // segments per chunk
  int64_t nchunk; // chunks per sequence
  // workspace offsets in bytes (each 256-byte aligned)
  size_t off_g, off_cp, off_bt, off_s, off_p, off_r, off_q, total;
};

inline SsdPlan make_ssd_plan(int64_t batch, int64_t seqlen, int64_t nheads) {
  SsdPlan p{};
  p.batch = batch;
  p.seqlen = seqlen;
  p.nheads = nheads;
  p.nsub = (seqlen + kQ - 1) / kQ;
  p.nseg = (p.nsub + kSeg - 1) / kSeg;
  int64_t spc = (p.nseg * batch * nheads + kTargetGroups / 2) / kTargetGroups;
  if (spc < 1) spc = 1;
  if (spc > p.nseg) spc = p.nseg;
  p.spc = spc;
  p.nchunk = (p.nseg + spc - 1) / spc;
  const size_t tile = static_cast<size_t>(batch) * p.nsub * kQ * kState * 2;  // bf16 [Q][N] per run
  const size_t gt = static_cast<size_t>(batch) * p.nsub * kQ * kQ * 4;       // fp32 [Q][Q] per run
  const size_t items = static_cast<size_t>(batch) * p.nchunk * nheads;
  size_t off = 0;
  p.off_g = off;  off = align256(off + gt);
  p.off_cp = off; off = align256(off + tile);
  p.off_bt = off; off = align256(off + tile);
  p.off_s = off;  off = align256(off + items * 2 * kStateFloats * sizeof(float));
  p.off_p = off;  off = align256(off + items * sizeof(float));
  p.off_r = off;  off = align256(off + items * static_cast<size_t>(spc - 1) * kStateFloats * sizeof(float));
  p.off_q = off;  off = align256(off + items * static_cast<size_t>(spc) * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace ssd
}  // namespace bimamba
