/*
 * bimamba.h - C ABI of the MI355X (gfx950) bidirectional selective-scan library.
 *
 * The operation is the bidirectional Mamba (S6) mixer scan of "DiffuMamba:
 * High-Throughput Diffusion LMs with Mamba Backbone" (arXiv v4):
 *   - Section 3.2, eq. (4): forward recurrence  h_i = A_f * h_{i-1} + B_f * x_i, i = 1..L
 *   - Section 3.2, eq. (5): reverse recurrence  h_i = A_b * h_{i+1} + B_b * x_i, i = L..1
 *   - Section 3.2, eq. (6): the two directions are summed.
 *   - Section 2 (state-space models): the SSM is selective, i.e. input-conditioned.
 *   - Appendix C, Table 12 caption: the input projection supplies the gate z,
 *     the step dt, B, C and a per-channel bias on dt.
 * with the selective discretisation written out per channel d, state n, token t:
 *   delta[t,d] = softplus(dt[t,d] + dt_bias[d])
 *   abar       = exp(delta[t,d] * A[d,n])
 *   h_fwd[t]   = abar * h_fwd[t-1] + delta[t,d] * x[t,d] * B[t,n]     (h_fwd[-1] = 0)
 *   h_rev[t]   = abar * h_rev[t+1] + delta[t,d] * x[t,d] * B[t,n]     (h_rev[L]  = 0)
 *   y_dir[t,d] = sum_n C[t,n] * h_dir[t,d,n] + D[d] * x[t,d]
 *   out[t,d]   = (y_fwd + y_rev) * z * sigmoid(z)
 * Both directions use one set of (A, D, dt_bias) and one (x, dt, B, C).
 *
 * Conventions common to every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or synchronises; work is enqueued on `stream` (0 = the
 *     null stream) and the call returns after enqueue.  A fault inside a kernel
 *     surfaces at the caller's next synchronisation.
 *   - Layouts are dense and row-major: x, dt, z, out are [batch, seqlen, d_inner]
 *     (channels contiguous); B and C are [batch, seqlen, d_state] (one B_t and
 *     one C_t per token, shared by all channels); A is [d_inner, d_state] fp32;
 *     D and dt_bias are [d_inner] fp32.  Base pointers must be 16-byte aligned.
 *   - io_dtype (a bimamba_dtype) applies to x, dt, z, B, C and out.  A, D,
 *     dt_bias, block states and every internal state are fp32; out is rounded
 *     to nearest even when io_dtype is BF16.
 *   - D == NULL means D = 0; dt_bias == NULL means dt_bias = 0; z may be NULL
 *     only together with BIMAMBA_FLAG_NO_GATE.  Inputs are read-only; out and
 *     the workspace must not overlap any input or each other (such a call is
 *     rejected with BIMAMBA_ERR_INVALID_ARGUMENT).
 *   - Supported shapes: 1 <= batch <= 65535, seqlen/block_len >= 1, d_inner a
 *     positive multiple of 64, 1 <= d_state <= 16, and the kernels' 32-bit
 *     buffer offsets: 16 * d_inner * element size and d_state * d_inner * 4 + 256
 *     bytes at most 2^31 - 1 (d_inner <= 33554368 at d_state 16); anything else
 *     returns BIMAMBA_ERR_UNSUPPORTED (unsupported values) or
 *     BIMAMBA_ERR_INVALID_ARGUMENT (non-positive sizes).
 *   - All arguments are validated before any HIP call, so a rejected call has
 *     no side effect.  Launch failures return BIMAMBA_ERR_HIP.
 *   - Calls are re-entrant; the library keeps no mutable global state.
 */
#ifndef BIMAMBA_H
#define BIMAMBA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BIMAMBA_OK = 0,
  BIMAMBA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad flag combination, misaligned pointer */
  BIMAMBA_ERR_UNSUPPORTED = 2,        /* shape or dtype outside the supported set */
  BIMAMBA_ERR_WORKSPACE_TOO_SMALL = 3,
  BIMAMBA_ERR_HIP = 4,                /* a HIP launch returned an error */
  BIMAMBA_ERR_SCRATCH_TOO_SMALL = 5   /* bimamba_scan_fwd_noalloc: the problem needs more than 256 MiB */
} bimamba_status;

typedef enum { BIMAMBA_F32 = 0, BIMAMBA_BF16 = 1 } bimamba_dtype;

enum {
  BIMAMBA_FLAG_NO_GATE = 1u,  /* out = y_fwd + y_rev, no SiLU(z) factor (z may be NULL) */
  BIMAMBA_FLAG_FWD_ONLY = 2u, /* keep only the forward direction, eq. (4)            */
  BIMAMBA_FLAG_REV_ONLY = 4u, /* keep only the reverse direction, eq. (5)            */
  BIMAMBA_FLAG_NO_SILU = 16u  /* short convolution only: return the filter output without SiLU */
};

/* Library version, (major << 16) | (minor << 8) | patch. */
int bimamba_version(void);

/* Static English text for a status code; never NULL. */
const char* bimamba_status_string(int status);

/* Bytes of device workspace bimamba_scan_fwd needs for this shape (a pure host
 * computation, no HIP call).  Returns 0 for an unsupported shape. */
size_t bimamba_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state);

/* Full-sequence bidirectional scan, Section 3.2 eq. (4)-(6): every token sees
 * the whole sequence in both directions.  out[b,t,d] as defined above.
 * workspace: caller-owned device memory of at least
 * bimamba_scan_fwd_workspace_bytes(...) bytes, 256-byte aligned; its contents
 * on entry are ignored and on exit are unspecified.  Two calls that overlap in
 * time must not share a workspace. */
int bimamba_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* dt_bias, void* out,
                     int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                     int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* One stage of bimamba_scan_fwd, for callers that schedule other work between
 * the stages or attribute time per stage.  stage 0 = chunk summaries (reads
 * B, C into an fp32 table in the workspace, then x, dt; writes the workspace),
 * 1 = carries across chunks (workspace only), 2 = output (reads x, dt, z and
 * the workspace; writes out).  Calling
 * stages 0, 1, 2 in this order on one stream with the same arguments and
 * workspace produces exactly what one bimamba_scan_fwd call produces.  Any
 * other stage value returns BIMAMBA_ERR_INVALID_ARGUMENT.  Arguments and
 * their checks are those of bimamba_scan_fwd. */
int bimamba_scan_fwd_stage(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, void* out,
                           int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                           int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* bimamba_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is the library's own
 * fixed device array of 256 MiB (each GPU the library runs on holds one copy
 * until the process ends); the call allocates and frees nothing.  A shape
 * whose bimamba_scan_fwd_workspace_bytes exceeds 256 MiB (268435456 bytes;
 * e.g. L * d_inner above about 2^25 at d_state 16) returns
 * BIMAMBA_ERR_SCRATCH_TOO_SMALL, checked before any HIP call.  All other
 * arguments, checks and results are those of bimamba_scan_fwd (bit for bit).
 * Every call on one GPU uses that GPU's one array: two calls that overlap in
 * time on the same GPU (different streams, or host threads without ordering)
 * race and both produce garbage; calls ordered on one stream are safe.  The
 * array's contents are not cleared between calls (nothing in it needs to start
 * at zero).  The first call on each device looks up the array's address there
 * (hipGetSymbolAddress with that device current). */
int bimamba_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* dt_bias, void* out,
                             int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                             int io_dtype, uint32_t flags, hipStream_t stream);

/* Bidirectional scan with untied directions: the forward and the reverse
 * scans are two separate selective-SSM layers, each with its own input
 * projection outputs (x, dt, B, C, z) and parameters (A, D, dt_bias), as in the
 * paper (Section 3.2: two independent Mamba layers, eq. (4) with A_f, B_f, C_f
 * and eq. (5) with A_b, B_b, C_b; Section 4.1 / Table 8: weights of the two
 * directions are not tied).  Each direction keeps its own gate and output
 * (each feeds its own output projection, outside this library):
 *   out_f = (C_f . h_fwd + D_f * x_f) * SiLU(z_f),  h_fwd from set f, eq. (4)
 *   out_r = (C_r . h_rev + D_r * x_r) * SiLU(z_r),  h_rev from set r, eq. (5)
 * with the discretisation of bimamba_scan_fwd (delta = softplus(dt + dt_bias),
 * abar = exp(delta A), input delta x B).  With both sets equal, out_f + out_r
 * is the output of bimamba_scan_fwd.
 * Shapes, dtypes, alignment, optional D / dt_bias and the workspace (size from
 * bimamba_scan_fwd_workspace_bytes, used by the two passes in turn) are as for
 * bimamba_scan_fwd; flags may only be BIMAMBA_FLAG_NO_GATE (then z_f and z_r
 * may be NULL).  Neither output may overlap any tensor of either set, the other
 * output or the workspace, and the workspace may not overlap any tensor of
 * either set; a rejected call returns a status and enqueues nothing. */
int bimamba_scan_fwd_untied(const void* x_f, const void* dt_f, const float* A_f, const void* B_f, const void* C_f,
                            const float* D_f, const void* z_f, const float* dt_bias_f, void* out_f,
                            const void* x_r, const void* dt_r, const float* A_r, const void* B_r, const void* C_r,
                            const float* D_r, const void* z_r, const float* dt_bias_r, void* out_r,
                            int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype,
                            uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace bimamba_scan_block needs for this shape; 0 when the
 * block is short enough for the single-kernel path (no workspace needed). */
size_t bimamba_scan_block_workspace_bytes(int64_t batch, int64_t block_len, int64_t d_inner, int64_t d_state);

/* One block of block-cache decoding (Section 4.3, block-cache paragraph; also
 * the abstract of arXiv 2607.02805, which restricts the reverse scan to the
 * active block): the forward direction resumes from the cached state h_in,
 * the reverse direction starts from zero at the block's last token and never
 * looks past the block.  x, dt, z, B, C, out hold the block's block_len tokens.
 *   h_in : [batch, d_inner, d_state] fp32, the forward state before the block;
 *          NULL means zeros.
 *   h_out: [batch, d_inner, d_state] fp32, receives the forward state after the
 *          block's last token (the cache for the next block); NULL means do not
 *          write.  h_out may equal h_in (in-place commit) but must not
 *          otherwise overlap it, nor any input or out; h_in must not overlap
 *          out.  The flags select the directions summed into out; h_out is the
 *          forward state in every case.
 * workspace may be NULL when bimamba_scan_block_workspace_bytes returns 0;
 * otherwise neither h_in, h_out nor any input may overlap it. */
int bimamba_scan_block(const void* x, const void* dt, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias,
                       const float* h_in, float* h_out, void* out,
                       int64_t batch, int64_t block_len, int64_t d_inner, int64_t d_state,
                       int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ---- Mamba-2 (SSD) heads ------------------------------------------------
 * The mixer the paper actually runs is a bidirectional Mamba-2 layer (Section
 * 1; Appendix A Table 7: SSM head size 32 and state size 128; Appendix C
 * Table 12 and its caption: d_inner = 3840, d_state = 128, a per-head bias on
 * Delta).  Channels form nheads heads of headdim channels (channel c = h *
 * headdim + p); the transition is one scalar per (token, head):
 *   delta[t,h] = softplus(dt[t,h] + dt_bias[h]),  abar = exp(delta[t,h] * A[h])
 *   H_fwd[t]   = abar * H_fwd[t-1] + delta[t,h] * x[t,h,:] (outer) B[t,:]   (H_fwd[-1] = 0)
 *   H_rev[t]   = abar * H_rev[t+1] + delta[t,h] * x[t,h,:] (outer) B[t,:]   (H_rev[L]  = 0)
 *   y_dir[t,c] = sum_n C[t,n] * H_dir[t,h,p,n] + D[h] * x[t,c]
 *   out[t,c]   = (y_fwd + y_rev) * z * sigmoid(z)
 * (Section 3.2 eq. (4)-(6) with Mamba-2's scalar-per-head transition; B_t and
 * C_t are shared by all heads.)  The products inside each 64-token run run on
 * the matrix cores with bf16 operands and fp32 accumulation; every state is
 * carried in fp32.
 * Layouts: x, z, out [batch, seqlen, nheads * headdim]; dt [batch, seqlen,
 * nheads]; B, C [batch, seqlen, d_state]; A, D, dt_bias [nheads] fp32.
 * Supported: io_dtype BIMAMBA_BF16, headdim 32, d_state 128, 1 <= nheads <= 2^18,
 * seqlen >= 1, batch >= 1 (others return BIMAMBA_ERR_UNSUPPORTED).  x, z, out,
 * B and C must be 16-byte aligned, dt 2-byte aligned, A, D, dt_bias 4-byte
 * aligned.  Flags, D == NULL, dt_bias == NULL, z == NULL, ownership,
 * asynchrony and the no-overlap rules are as for bimamba_scan_fwd. */
size_t bimamba_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                       int64_t d_state);

int bimamba_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* dt_bias, void* out,
                    int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                    int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One stage of bimamba_ssd_fwd, for per-kernel timing: 0 tiles B and C, 1 the
 * chunk summaries, 2 the carry across chunks, 3 the output pass.  Running 0..3
 * in order with the same workspace equals one bimamba_ssd_fwd call. */
int bimamba_ssd_fwd_stage(int stage, const void* x, const void* dt, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* dt_bias, void* out,
                          int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                          int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Bytes of device workspace bimamba_ssd_block needs: 0 for blocks of at most
 * 64 tokens (one kernel), otherwise the same as a full call over block_len
 * tokens. */
size_t bimamba_ssd_block_workspace_bytes(int64_t batch, int64_t block_len, int64_t nheads, int64_t headdim,
                                         int64_t d_state);

/* One block of block-cache decoding with Mamba-2 heads (Section 4.3,
 * block-cache paragraph): the forward direction resumes from the cached state
 * h_in, the reverse direction starts from zero after the block's last token
 * and never looks past the block.  x, dt, z, B, C, out hold the block's
 * block_len tokens; everything else is as in bimamba_ssd_fwd.
 *   h_in : [batch, nheads, headdim, d_state] fp32 (state n of channel
 *          h*headdim + p at ((b*nheads + h)*headdim + p)*d_state + n), the
 *          forward state before the block; NULL means zeros.
 *   h_out: the same layout, receives the forward state after the block's last
 *          token (the cache of the next block); NULL means do not write.  It
 *          may equal h_in (in-place commit) but must not otherwise overlap it,
 *          nor any input, out or the workspace; h_in must not overlap out or
 *          the workspace.  With BIMAMBA_FLAG_REV_ONLY the forward state is not
 *          computed and h_out must be NULL (INVALID_ARGUMENT otherwise).
 * h_in and h_out are 4-byte aligned.  workspace may be NULL when
 * bimamba_ssd_block_workspace_bytes returns 0. */
int bimamba_ssd_block(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                      const void* z, const float* dt_bias, const float* h_in, float* h_out, void* out,
                      int64_t batch, int64_t block_len, int64_t nheads, int64_t headdim, int64_t d_state,
                      int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Mamba-2 layers with untied directions, each with its short convolution: the
 * bidirectional mixer as the paper runs it (Section 3.2: two independent
 * layers, the reverse one on the flipped sequence; Section 4.1 Table 8: the
 * directions' weights are not tied, convolution width 4; Appendix C Table 12:
 * the projection's xBC stream of conv_ch = d_inner + 2 d_state channels goes
 * through Conv1d before the scan, and the gate z and the step dt come from the
 * same projection).  For each direction's set (xbc, cw, cb, dt, A, D, z,
 * dt_bias, out), with P = headdim, N = d_state and channel c of the stream:
 *   u[t,c]  = silu(cb[c] + sum_k cw[c,k] * xbc[t-3+k, c])   forward set (causal)
 *   u[t,c]  = silu(cb[c] + sum_k cw[c,k] * xbc[t+3-k, c])   reverse set (anti-causal)
 *   (xbc = 0 outside the sequence; u is rounded to nearest even bf16, as when
 *   the convolution's output is stored before the scan)
 *   x = u[:, 0 : H*P], B = u[:, H*P : H*P+N], C = u[:, H*P+N : H*P+2N]
 *   out_f = (y_fwd(x, B, C) + D * x) * silu(z)   (bimamba_ssd_fwd's forward scan)
 *   out_r = (y_rev(x, B, C) + D * x) * silu(z)   (its reverse scan)
 * with each set's own dt [batch, seqlen, nheads], A, D, dt_bias [nheads] and
 * z [batch, seqlen, H*P].  cw == NULL skips the convolution (x, B, C are then
 * the stream itself); cb == NULL means no bias.  out_f or out_r may be NULL to
 * skip that layer (not both); its set's pointers are then not read.
 * Layouts: xbc [batch, seqlen, H*P + 2N] bf16, cw [H*P + 2N, 4] and cb
 * [H*P + 2N] fp32, out [batch, seqlen, H*P] bf16.  Shapes, dtype, heads and
 * D / dt_bias NULL are as for bimamba_ssd_fwd, and with a convolution one
 * batch element's stream must stay below 2^31 bytes (seqlen * (H*P + 2N) * 2
 * + 256, e.g. seqlen <= 262143 at 4096 channels); d_conv must be 4; flags may only
 * be BIMAMBA_FLAG_NO_GATE (then z may be NULL).  xbc, z and out 16-byte
 * aligned, dt 2-byte, the fp32 parameters 4-byte.  The workspace
 * (bimamba_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state)
 * bytes, 256-byte aligned) is used by the two layers in turn.  Neither output
 * may overlap any tensor of either set, the other output or the workspace. */
int bimamba_ssd_conv_untied(const void* xbc_f, const float* cw_f, const float* cb_f, const void* dt_f,
                            const float* A_f, const float* D_f, const void* z_f, const float* dt_bias_f, void* out_f,
                            const void* xbc_r, const float* cw_r, const float* cb_r, const void* dt_r,
                            const float* A_r, const float* D_r, const void* z_r, const float* dt_bias_r, void* out_r,
                            int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t d_state,
                            int64_t d_conv, int io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---- Short causal / anti-causal convolution ------------------------------
 * Each direction of the mixer runs a depthwise Conv1d of width d_conv = 4
 * ahead of its scan (Appendix C Table 12: conv_ch = 4096 channels at the 1.3B
 * shape, one multiply-add per token, channel and tap; Section 4.1 Table 8:
 * width 4, directions not tied); the reverse layer is the forward layer on
 * the flipped sequence (Section 3.2).  Per channel c and token t:
 *   out_f[t,c] = silu(b_f[c] + sum_k w_f[c,k] * u[t-3+k, c])     (causal)
 *   out_r[t,c] = silu(b_r[c] + sum_k w_r[c,k] * u[t+3-k, c])     (anti-causal)
 * with u = 0 outside the sequence.  Both directions come from one read of u.
 * Layouts: u, out_f, out_r [batch, seqlen, channels] (io_dtype); w_f, w_r
 * [channels, d_conv] fp32; b_f, b_r [channels] fp32 or NULL (= 0).  For tied
 * weights pass the same pointers twice.  out_f or out_r may be NULL to skip
 * that direction (not both); its weights may then be NULL too.
 * Supported: d_conv 4, channels a multiple of 4 and at most 4194304 (2^22),
 * batch at most 65535, io_dtype F32 or BF16 (fp32
 * arithmetic, round to nearest even for bf16).  u, outputs and caches must be
 * aligned to 4 elements (8 bytes bf16, 16 bytes fp32), weights and biases to 4
 * bytes.  flags: 0 or BIMAMBA_FLAG_NO_SILU.  Outputs must not overlap any
 * input, each other or a cache.  Ownership and asynchrony as above. */
int bimamba_conv1d_bidir(const void* u, const float* w_f, const float* b_f, const float* w_r, const float* b_r,
                         void* out_f, void* out_r, int64_t batch, int64_t seqlen, int64_t channels,
                         int64_t d_conv, int io_dtype, uint32_t flags, hipStream_t stream);

/* The same for one block of block decoding (Section 4.3, block-cache
 * paragraph): the causal filter reads the 3 tokens before the block from
 * cache_in ([batch, 3, channels], io_dtype, oldest first; NULL = zeros) and the
 * anti-causal filter sees zeros past the block's last token.  cache_out
 * ([batch, 3, channels]; NULL = not written) receives the last 3 tokens of
 * (cache_in, block), the cache of the next block; it may equal cache_in
 * (in-place commit) but must not otherwise overlap it. */
int bimamba_conv1d_block(const void* u, const float* w_f, const float* b_f, const float* w_r, const float* b_r,
                         const void* cache_in, void* cache_out, void* out_f, void* out_r, int64_t batch,
                         int64_t block_len, int64_t channels, int64_t d_conv, int io_dtype, uint32_t flags,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BIMAMBA_H */
