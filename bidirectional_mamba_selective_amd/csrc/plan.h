// Host-side decomposition of a scan into chunks and sub-chunks, and the
// layout of the caller-provided workspace.  Pure host code: no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace bimamba {

// Tokens per register-resident sub-chunk of the output kernel.  The summary
// kernel stores the reverse state at every sub-chunk boundary.
constexpr int64_t kSub = 16;
// Channels per wavefront (one channel per lane).
constexpr int64_t kLanes = 64;
// Wavefronts the chunking aims to give the summary and output kernels (four per
// SIMD on a 256-CU part).
constexpr int64_t kTargetWaves = 4096;
// Longest block the single-kernel block path handles (it needs no workspace).
constexpr int64_t kBlockFusedMax = 128;

struct Plan {
  int64_t batch, seqlen, d_inner, d_state;
  int64_t chunk;   // tokens per chunk (multiple of kSub)
  int64_t nchunk;  // chunks per sequence
  int64_t nsub;    // sub-chunks per full chunk (chunk / kSub)
  int64_t ntile;   // kSub-token tiles per sequence (chunks start on tile boundaries)
  // workspace offsets in bytes (each 256-byte aligned)
  size_t off_sf, off_sr, off_p, off_cf, off_cr, off_r, off_sig, off_a2t, off_bct, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

inline Plan make_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  Plan p{};
  p.batch = batch;
  p.seqlen = seqlen;
  p.d_inner = d_inner;
  p.d_state = d_state;
  const int64_t row_waves = batch * (d_inner / kLanes);
  int64_t want_chunks = (kTargetWaves + row_waves - 1) / row_waves;
  if (want_chunks < 1) want_chunks = 1;
  int64_t chunk = (seqlen + want_chunks - 1) / want_chunks;
  chunk = ((chunk + kSub - 1) / kSub) * kSub;
  if (chunk < kSub) chunk = kSub;
  p.chunk = chunk;
  p.nchunk = (seqlen + chunk - 1) / chunk;
  p.nsub = chunk / kSub;
  p.ntile = (seqlen + kSub - 1) / kSub;
  const size_t state = static_cast<size_t>(batch) * p.nchunk * d_state * d_inner * sizeof(float);
  const size_t bound = static_cast<size_t>(batch) * p.nchunk * p.nsub * d_state * d_inner * sizeof(float);
  const size_t sig = static_cast<size_t>(batch) * p.nchunk * p.nsub * d_inner * sizeof(float);
  size_t off = 0;
  p.off_sf = off; off = align256(off + state);
  p.off_sr = off; off = align256(off + state);
  p.off_p = off;  off = align256(off + state);
  p.off_cf = off; off = align256(off + state);
  p.off_cr = off; off = align256(off + state);
  p.off_r = off;  off = align256(off + bound);
  p.off_sig = off; off = align256(off + sig);
  p.off_a2t = off; off = align256(off + static_cast<size_t>(d_state) * d_inner * sizeof(float));
  // B and C in fp32, per tile and state: kSub values of B then kSub of C
  p.off_bct = off; off = align256(off + static_cast<size_t>(batch) * p.ntile * d_state * 2 * kSub * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace bimamba
