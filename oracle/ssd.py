"""Plain fp64 CPU oracle for the bidirectional Mamba-2 (SSD) scan.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
table or constant with the HIP library.

Sources (page = "DiffuMamba: High-Throughput Diffusion LMs with Mamba
Backbone", arXiv HTML v4):
  * Section 1 "Introduction" and the conclusion: the mixers are bidirectional
    Mamba-2 layers.
  * Appendix A, Table 7: SSM head size 32 and state size 128 at every scale.
  * Appendix C, Table 12 and its caption: d_inner = 3840 and d_state = 128 for
    the 1.3B model; the input projection yields the gate, Delta, B, C and a
    per-head bias on Delta; the scan costs one update and one readout per
    (token, channel, state) and direction.
  * Section 3.2, eq. (4)-(6): one recurrence left to right, one right to left,
    the two streams summed.
The pages name Mamba-2 but print none of its equations.  The reading taken
here is the same recurrence as eq. (4)/(5) with the structure Mamba-2 is
known for: the channels are split into heads of headdim channels, A, D and
the Delta bias are one scalar per head, Delta is one value per (token, head),
and B_t, C_t are shared by all heads (one group, as the Table 12 projection
width implies):
  Delta[t, h]   = softplus(dt[t, h] + dt_bias[h])
  abar[t, h]    = exp(Delta[t, h] * A[h])                       (a scalar)
  H_t[h]        = abar[t, h] * H_{t-1}[h] + Delta[t, h] * x_t[h, :] (outer) B_t
  G_t[h]        = abar[t, h] * G_{t+1}[h] + Delta[t, h] * x_t[h, :] (outer) B_t
  y_dir[t, h, p] = sum_n C_t[n] * state_t[h, p, n] + D[h] * x_t[h, p]
  out           = (y_fwd + y_rev) * z * sigmoid(z)
with H, G of shape [headdim, d_state] per head, H_{-1} = G_L = 0 (for one block
of block-cache decoding, H_{-1} is the cached state; see ssd_scan_block).

Shapes: x, z, out are [batch, L, nheads * headdim] with channel c = h *
headdim + p; dt is [batch, L, nheads]; B, C are [batch, L, d_state]; A, D and
dt_bias are [nheads].  Inputs are upcast exactly to float64 and the result
is returned in float64 with no rounding emulated.
"""
from __future__ import annotations

import numpy as np

from .scan import silu, softplus

__all__ = ["ssd_discretise", "ssd_forward_scan", "ssd_reverse_scan", "ssd_scan_fwd", "ssd_scan_block"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def ssd_discretise(dt, dt_bias):
    """Per-(token, head) step size Delta = softplus(dt + dt_bias[h]).

    Appendix C, Table 12 caption: Delta and a per-head bias come out of the
    input projection.  dt is [batch, L, nheads].
    """
    dt = _f64(dt)
    v = dt if dt_bias is None else dt + _f64(dt_bias)[None, None, :]
    return softplus(v)


def _heads(x, nheads):
    x = _f64(x)
    nb, L, nc = x.shape
    if nc % nheads:
        raise ValueError("channel count is not a multiple of the head count")
    return x.reshape(nb, L, nheads, nc // nheads)


def ssd_forward_scan(delta, xh, A, B, C, h0=None):
    """Left-to-right recurrence (eq. (4) with a scalar transition per head).

    delta [batch, L, H]; xh [batch, L, H, P]; A [H]; B, C [batch, L, N].
    H_t = exp(delta_t A) H_{t-1} + delta_t x_t (outer) B_t, readout C_t . H_t.
    Returns (y [batch, L, H, P], state after the last token [batch, H, P, N]).
    """
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    nb, L, nh, hp = xh.shape
    h = np.zeros((nb, nh, hp, B.shape[-1])) if h0 is None else _f64(h0).copy()
    y = np.empty((nb, L, nh, hp))
    for t in range(L):
        abar = np.exp(delta[:, t, :] * A[None, :])
        u = delta[:, t, :, None] * xh[:, t]
        h = abar[:, :, None, None] * h + u[:, :, :, None] * B[:, t, None, None, :]
        y[:, t] = np.sum(h * C[:, t, None, None, :], axis=-1)
    return y, h


def ssd_reverse_scan(delta, xh, A, B, C, g0=None):
    """Right-to-left recurrence (eq. (5) with a scalar transition per head).

    G_t = exp(delta_t A) G_{t+1} + delta_t x_t (outer) B_t for t = L-1 .. 0,
    starting from g0 (zeros when None); step t uses the transition of token t
    itself.  Returns (y, state after token 0).
    """
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    nb, L, nh, hp = xh.shape
    g = np.zeros((nb, nh, hp, B.shape[-1])) if g0 is None else _f64(g0).copy()
    y = np.empty((nb, L, nh, hp))
    for t in range(L - 1, -1, -1):
        abar = np.exp(delta[:, t, :] * A[None, :])
        u = delta[:, t, :, None] * xh[:, t]
        g = abar[:, :, None, None] * g + u[:, :, :, None] * B[:, t, None, None, :]
        y[:, t] = np.sum(g * C[:, t, None, None, :], axis=-1)
    return y, g


def ssd_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, *, gate=True, fwd=True, rev=True):
    """Full-sequence bidirectional Mamba-2 scan (Section 3.2, eq. (4)-(6)).

    out = (y_fwd + y_rev) * silu(z), each direction y = C . state + D[h] * x.
    gate=False drops the SiLU factor; fwd/rev select the directions kept.
    D=None and dt_bias=None mean zero.  The head count is len(A).
    """
    return ssd_scan_block(x, dt, A, B, C, D, z, dt_bias, None, gate=gate, fwd=fwd, rev=rev)[0]


def ssd_scan_block(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, *, gate=True, fwd=True, rev=True):
    """One block of block-cache decoding with Mamba-2 heads: (out, h_next).

    Section 4.3 (block-cache paragraph): the left-to-right state is cached from
    the blocks before and carried into this one, while the right-to-left state
    stays inside the active block.  So the forward recurrence starts from h0
    ([batch, nheads, headdim, d_state]; zeros when None), the reverse one from
    zero after the block's last token, and h_next is the forward state after
    the block's last token (the cache of the next block) whatever directions
    out keeps.  With h0 = None this is the full-sequence scan.
    """
    if gate and z is None:
        raise ValueError("z is required when the gate is applied")
    A = _f64(A)
    nh = A.shape[0]
    xh = _heads(x, nh)
    delta = ssd_discretise(dt, dt_bias)
    if delta.shape[-1] != nh:
        raise ValueError("dt must hold one value per (token, head)")
    y_f, h_next = ssd_forward_scan(delta, xh, A, B, C, h0)
    out = np.zeros_like(xh)
    for keep, y in ((fwd, y_f), (rev, ssd_reverse_scan(delta, xh, A, B, C)[0] if rev else None)):
        if not keep:
            continue
        out = out + y
        if D is not None:
            out = out + _f64(D)[None, None, :, None] * xh
    out = out.reshape(_f64(x).shape)
    if gate:
        out = out * silu(z)
    return out, h_next
