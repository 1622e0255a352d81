"""Plain fp64 CPU oracle for the short causal / anti-causal depthwise convolution.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
table or constant with the HIP library.

Sources (page = "DiffuMamba: High-Throughput Diffusion LMs with Mamba
Backbone", arXiv HTML v4):
  * Appendix C, Table 12: each direction of the Mamba-2 layer runs a short
    Conv1d of width d_conv = 4 over conv_ch = 4096 channels, one
    multiply-add per (token, channel, tap); Table 8 (Section 4.1) lists the
    conv width 4 and says the two directions' weights are not tied.
  * Section 3.2: the bidirectional mixer is described through causal and
    anti-causal one-dimensional convolutions; the reverse layer is the forward
    layer applied to the time-reversed sequence.
  * Section 4.3 (block-cache paragraph): in block decoding the forward
    direction carries a cache from earlier blocks while the reverse direction
    stays inside the active block.
The pages do not print the convolution itself.  The reading taken here is the
Mamba convention: a depthwise (per-channel) filter of width K with left
padding K-1, a per-channel bias and a SiLU activation:
  fwd[t, c] = silu(b_f[c] + sum_{k=0}^{K-1} w_f[c, k] * u[t - (K-1) + k, c])
  rev[t, c] = silu(b_r[c] + sum_{k=0}^{K-1} w_r[c, k] * u[t + (K-1) - k, c])
(rev is the forward filter run on the flipped sequence and flipped back), with
u = 0 outside the sequence, or, in block decoding, u before the block taken
from the cached last K-1 tokens of the previous blocks and u after the block
taken as 0.

Shapes: u, fwd, rev are [batch, L, channels]; w_f, w_r are [channels, K];
b_f, b_r are [channels] (None = 0); the cache is [batch, K-1, channels],
oldest token first.  Inputs are upcast exactly to float64; no rounding is
emulated.
"""
from __future__ import annotations

import numpy as np

from .scan import silu

__all__ = ["conv_causal", "conv_anticausal", "conv_bidir", "conv_block"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def conv_causal(u, w, b=None, cache=None, *, act=True):
    """Depthwise causal filter (Table 12's Conv1d, left padding K-1).

    out[t] = b + sum_k w[:, k] * u[t - (K-1) + k]; positions before the
    sequence read the cache (its last K-1 tokens, oldest first) or zero.
    act=False returns the pre-activation.
    """
    u = _f64(u)
    w = _f64(w)
    nb, L, nc = u.shape
    K = w.shape[1]
    pre = np.zeros((nb, K - 1, nc)) if cache is None else _f64(cache)
    ext = np.concatenate([pre, u], axis=1)  # ext[K-1 + t] = u[t]
    out = np.zeros((nb, L, nc)) if b is None else np.broadcast_to(_f64(b), (nb, L, nc)).copy()
    for t in range(L):
        for k in range(K):
            out[:, t, :] += w[None, :, k] * ext[:, t + k, :]
    return silu(out) if act else out


def conv_anticausal(u, w, b=None, *, act=True):
    """The same filter run on the time-reversed sequence (Section 3.2's reverse layer).

    out[t] = b + sum_k w[:, k] * u[t + (K-1) - k]; positions past the end read zero.
    """
    u = _f64(u)
    w = _f64(w)
    nb, L, nc = u.shape
    K = w.shape[1]
    ext = np.concatenate([u, np.zeros((nb, K - 1, nc))], axis=1)
    out = np.zeros((nb, L, nc)) if b is None else np.broadcast_to(_f64(b), (nb, L, nc)).copy()
    for t in range(L):
        for k in range(K):
            out[:, t, :] += w[None, :, k] * ext[:, t + (K - 1) - k, :]
    return silu(out) if act else out


def conv_bidir(u, w_f, b_f, w_r, b_r, *, act=True):
    """Both directions of the mixer's short convolution over the whole sequence: (fwd, rev)."""
    return conv_causal(u, w_f, b_f, act=act), conv_anticausal(u, w_r, b_r, act=act)


def conv_block(u, w_f, b_f, w_r, b_r, cache=None, *, act=True):
    """One block of block decoding: (fwd, rev, cache_out).

    The forward filter reads the cached last K-1 tokens before the block (zeros
    when None); the reverse filter sees zeros past the block's last token.
    cache_out holds the last K-1 tokens of (cache, block), oldest first: the
    cache the next block starts from.
    """
    u = _f64(u)
    nb, L, nc = u.shape
    K = _f64(w_f).shape[1]
    pre = np.zeros((nb, K - 1, nc)) if cache is None else _f64(cache)
    fwd = conv_causal(u, w_f, b_f, pre, act=act)
    rev = conv_anticausal(u, w_r, b_r, act=act)
    cache_out = np.concatenate([pre, u], axis=1)[:, -(K - 1):, :].copy()
    return fwd, rev, cache_out
