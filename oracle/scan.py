"""Plain fp64 CPU oracle for the bidirectional selective (S6) scan.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
table or constant with the HIP library.

Sources (page = "DiffuMamba: High-Throughput Diffusion LMs with Mamba
Backbone", arXiv HTML v4, unless noted):
  * Section 3.2 "Diffusion Mamba Language Models", eq. (4) and (5) (restated
    in Appendix A.1 as eq. (7) and (8)): a forward recurrence over i = 1..L and
    a reverse recurrence over i = L..1, one per direction.
  * Section 3.2, eq. (6) (Appendix A.1 eq. (9)): the two directional streams
    are fused by a plain sum.
  * Section 2 "Related Work", paragraph on state-space models: the SSM is
    input-conditioned ("selective"), i.e. the step size and the B, C vectors
    depend on the token.
  * Appendix C, Table 12 caption: the projection in front of the SSM yields a
    gate, the step size Delta, B, C and a per-channel bias on Delta; the scan
    costs one state update and one readout per (token, channel, state).
  * Section 4.3 "Inference Throughput" (block-cache paragraph) and the
    abstract of "Training Hybrid Block Diffusion Language Models with Partial
    Bidirectionality" (arXiv 2607.02805): in block decoding the forward state
    is carried across blocks while the reverse scan stays inside the active
    block.

The pages leave the discretisation, the readout and the gate open.  The
readings taken here (listed with reasons in the design notes of the
repository) are:
  Delta = softplus(dt + dt_bias)           (bias added before the activation)
  abar  = exp(Delta * A)                   (zero-order hold on A)
  ubar  = Delta * x                        (Euler step on B: input term Delta*B*x)
  h_t   = abar_t * h_{t-1} + ubar_t * B_t  (forward, h_{-1} = 0)
  g_t   = abar_t * g_{t+1} + ubar_t * B_t  (reverse, g_L = 0; step t uses abar_t)
  y_dir = C_t . state_t + D * x_t          (each direction is a full layer)
  out   = (y_fwd + y_rev) * z * sigmoid(z) (one SiLU gate on the sum)

Shapes: x, dt, z, out are [batch, L, d_inner]; B, C are [batch, L, d_state]
(one B_t, C_t per token, shared by all channels); A is [d_inner, d_state];
D and dt_bias are [d_inner].  Every input is upcast exactly to float64 and the
result is returned in float64 with no rounding emulated.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "softplus",
    "silu",
    "discretise",
    "forward_scan",
    "reverse_scan",
    "scan_fwd",
    "scan_block",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def softplus(v):
    """log(1 + e^v), evaluated stably as max(v, 0) + log1p(exp(-|v|)).

    The step-size activation applied to the biased Delta pre-activation
    (Appendix C, Table 12 caption: Delta and a per-head bias come out of the
    input projection; the activation itself is the plainest reading).
    """
    v = _f64(v)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def silu(z):
    """z * sigmoid(z) with a sign-split sigmoid that never overflows.

    The gate branch of the input projection (Appendix C, Table 12 caption).
    """
    z = _f64(z)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def discretise(x, dt, dt_bias):
    """Per-token step size and input term (selective SSM, Section 2).

    Returns (delta, ubar) of shape [batch, L, d_inner]:
      delta = softplus(dt + dt_bias),  ubar = delta * x.
    The per-state transition abar = exp(delta * A) is formed per step inside
    the scans so that the [batch, L, d_inner, d_state] tensor never exists.
    """
    x = _f64(x)
    dt = _f64(dt)
    v = dt if dt_bias is None else dt + _f64(dt_bias)[None, None, :]
    delta = softplus(v)
    return delta, delta * x


def forward_scan(delta, ubar, A, B, C, h0=None):
    """Forward recurrence, eq. (4) / (7), and its readout C_t . h_t.

    h_t = exp(delta_t * A) * h_{t-1} + ubar_t * B_t  for t = 0 .. L-1,
    starting from h0 (zeros when None).  Returns (y, h_last) with
    y[b, t, d] = sum_n C[b, t, n] * h_t[b, d, n] and h_last the state after
    the last token, shape [batch, d_inner, d_state].
    """
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    nb, L, nd = delta.shape
    ns = A.shape[1]
    h = np.zeros((nb, nd, ns)) if h0 is None else _f64(h0).copy()
    y = np.empty((nb, L, nd))
    for t in range(L):
        abar = np.exp(delta[:, t, :, None] * A[None, :, :])
        h = abar * h + ubar[:, t, :, None] * B[:, t, None, :]
        y[:, t, :] = np.sum(h * C[:, t, None, :], axis=-1)
    return y, h


def reverse_scan(delta, ubar, A, B, C, g0=None):
    """Reverse recurrence, eq. (5) / (8), and its readout C_t . g_t.

    g_t = exp(delta_t * A) * g_{t+1} + ubar_t * B_t  for t = L-1 .. 0, starting
    from g0 (zeros when None) after the last token.  Step t uses the
    transition of token t itself, the same one the forward direction uses.
    Returns (y, g_first) with g_first the state after token 0.
    """
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    nb, L, nd = delta.shape
    ns = A.shape[1]
    g = np.zeros((nb, nd, ns)) if g0 is None else _f64(g0).copy()
    y = np.empty((nb, L, nd))
    for t in range(L - 1, -1, -1):
        abar = np.exp(delta[:, t, :, None] * A[None, :, :])
        g = abar * g + ubar[:, t, :, None] * B[:, t, None, :]
        y[:, t, :] = np.sum(g * C[:, t, None, :], axis=-1)
    return y, g


def _combine(y_f, y_r, x, D, z, gate):
    """Direction sum, eq. (6) / (9), skip term per direction, then the gate."""
    x = _f64(x)
    out = np.zeros_like(x)
    for y in (y_f, y_r):
        if y is None:
            continue
        out = out + y
        if D is not None:
            out = out + _f64(D)[None, None, :] * x
    if gate:
        out = out * silu(z)
    return out


def scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, *, gate=True, fwd=True, rev=True):
    """Full-sequence bidirectional scan (Section 3.2, eq. (4)-(6)).

    out = (y_fwd + y_rev) * silu(z), each direction y = C . state + D * x.
    gate=False drops the SiLU factor; fwd/rev select the directions kept.
    D=None and dt_bias=None mean zero.
    """
    if gate and z is None:
        raise ValueError("z is required when the gate is applied")
    delta, ubar = discretise(x, dt, dt_bias)
    y_f = forward_scan(delta, ubar, A, B, C)[0] if fwd else None
    y_r = reverse_scan(delta, ubar, A, B, C)[0] if rev else None
    return _combine(y_f, y_r, x, D, z, gate)


def scan_block(x, dt, A, B, C, D=None, z=None, dt_bias=None, h_in=None, *, gate=True, fwd=True, rev=True):
    """One block of block-cache decoding (Section 4.3, block-cache paragraph).

    The forward direction resumes from the cached state h_in (zeros when
    None); the reverse direction starts from zero at the block's last token
    and never looks past the block.  Returns (out, h_out) where h_out is the
    forward state after the block's last token, the cache the next block
    resumes from.  fwd/rev select the directions summed into out; h_out is the
    forward state in every case.
    """
    if gate and z is None:
        raise ValueError("z is required when the gate is applied")
    delta, ubar = discretise(x, dt, dt_bias)
    y_f, h_out = forward_scan(delta, ubar, A, B, C, h_in)
    y_r = reverse_scan(delta, ubar, A, B, C)[0] if rev else None
    out = _combine(y_f if fwd else None, y_r, x, D, z, gate)
    return out, h_out


def scan_fwd_untied(fwd_set, rev_set, *, gate=True):
    """Bidirectional scan with untied directions.

    The paper runs the two directions as two independent Mamba layers
    (Section 3.2; eq. (4) carries A_f, B_f, C_f and eq. (5) A_b, B_b, C_b), and
    its Table 8 (Section 4.1) lists the weights of the two directions as not
    tied.  Each direction is then a complete layer with its own projection
    outputs (x, dt, B, C, z) and parameters (A, D, dt_bias); each keeps its own
    gate and output, because each feeds its own output projection before the
    sum of eq. (6).  fwd_set and rev_set are dicts with keys x, dt, A, B, C and
    optionally D, z, dt_bias.  Returns (out_f, out_r).
    """
    keys = ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")
    f = [fwd_set.get(k) for k in keys]
    r = [rev_set.get(k) for k in keys]
    out_f = scan_fwd(*f, gate=gate, fwd=True, rev=False)
    out_r = scan_fwd(*r, gate=gate, fwd=False, rev=True)
    return out_f, out_r
