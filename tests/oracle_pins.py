"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the oracle itself.

Each pin takes an implementation object exposing ``scan_fwd`` and
``scan_block`` with the oracle's signatures and returns ``(ok, detail)``.
The expected values are computed here independently of the oracle's code
(different formulas for softplus and the gate, closed forms, np.convolve,
brute-force sums), so a mistake in the oracle shows up as a failed pin.

Section and equation numbers refer to "DiffuMamba: High-Throughput Diffusion
LMs with Mamba Backbone" (arXiv v4).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _softplus(v):
    # independent formula: log(e^0 + e^v)
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


def _silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-np.clip(z, -700, 700)))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b.ravel())
    num = np.linalg.norm((a - b).ravel())
    return num / den if den > 0 else num


def _rand_case(rng, nb, L, nd, ns, a_range=(0.2, 3.0)):
    x = rng.standard_normal((nb, L, nd))
    dt = 0.5 * rng.standard_normal((nb, L, nd))
    z = rng.standard_normal((nb, L, nd))
    B = rng.standard_normal((nb, L, ns))
    C = rng.standard_normal((nb, L, ns))
    A = -rng.uniform(*a_range, size=(nd, ns))
    D = rng.standard_normal(nd)
    dt_bias = rng.uniform(-3.0, 0.5, size=nd)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias)


def brute_force(case, fwd=True, rev=True, gate=True, h_in=None):
    """Unrolled closed form of eq. (4)-(6) by triple loop (O(L^2 * D * N)).

    y_fwd[t] = sum_{s<=t} sum_n C[t,n] exp(A[d,n] * sum_{r=s+1..t} Delta_r) Delta_s B[s,n] x_s
               (+ sum_n C[t,n] exp(A[d,n] * sum_{r=0..t} Delta_r) h_in[d,n])
    y_rev[t] = sum_{s>=t} sum_n C[t,n] exp(A[d,n] * sum_{r=t..s-1} Delta_r) Delta_s B[s,n] x_s
    each plus D x_t, summed, times silu(z_t).
    """
    x, dt, A, B, C = (np.asarray(case[k], dtype=np.float64) for k in ("x", "dt", "A", "B", "C"))
    nb, L, nd = x.shape
    ns = A.shape[1]
    bias = case.get("dt_bias")
    dl = _softplus(dt + (0.0 if bias is None else np.asarray(bias)[None, None, :]))
    Dv = case.get("D")
    out = np.zeros((nb, L, nd))
    for b in range(nb):
        for d in range(nd):
            for t in range(L):
                acc = 0.0
                if fwd:
                    for s in range(t + 1):
                        seg = dl[b, s + 1:t + 1, d].sum()
                        for n in range(ns):
                            acc += C[b, t, n] * math.exp(A[d, n] * seg) * dl[b, s, d] * B[b, s, n] * x[b, s, d]
                    if h_in is not None:
                        seg = dl[b, 0:t + 1, d].sum()
                        for n in range(ns):
                            acc += C[b, t, n] * math.exp(A[d, n] * seg) * h_in[b, d, n]
                    if Dv is not None:
                        acc += Dv[d] * x[b, t, d]
                if rev:
                    for s in range(t, L):
                        seg = dl[b, t:s, d].sum()
                        for n in range(ns):
                            acc += C[b, t, n] * math.exp(A[d, n] * seg) * dl[b, s, d] * B[b, s, n] * x[b, s, d]
                    if Dv is not None:
                        acc += Dv[d] * x[b, t, d]
                out[b, t, d] = acc
    if gate:
        out = out * _silu(case["z"])
    return out


def _call(impl, case, **kw):
    return impl.scan_fwd(case["x"], case["dt"], case["A"], case["B"], case["C"], case.get("D"), case.get("z"),
                         case.get("dt_bias"), **kw)


def pin_brute_force(impl, seeds=range(6)):
    """P1: the recurrences equal their unrolled closed form (tiny sizes, many seeds)."""
    worst = 0.0
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        case = _rand_case(rng, 1 + seed % 2, 5 + 2 * seed, 1 + seed % 3, 1 + seed % 4)
        for fwd, rev, gate in ((True, True, True), (True, False, False), (False, True, False)):
            got = _call(impl, case, fwd=fwd, rev=rev, gate=gate)
            want = brute_force(case, fwd=fwd, rev=rev, gate=gate)
            worst = max(worst, _rel(got, want))
    return worst < 1e-12, f"max rel err {worst:.3e}"


def pin_flip(impl):
    """P2: the reverse scan is the forward scan of the time-reversed input."""
    rng = np.random.default_rng(7)
    case = _rand_case(rng, 2, 40, 3, 4)
    flipped = dict(case)
    for k in ("x", "dt", "z", "B", "C"):
        flipped[k] = case[k][:, ::-1, :].copy()
    rev = _call(impl, case, fwd=False, rev=True, gate=False)
    fwd_of_flip = _call(impl, flipped, fwd=True, rev=False, gate=False)[:, ::-1, :]
    err = _rel(rev, fwd_of_flip)
    return err < 1e-13, f"rel err {err:.3e}"


def pin_delta_to_zero(impl):
    """P3: dt_bias = -60 makes Delta ~ 1e-26, so out = 2 D x silu(z) and, with D = 0, out ~ 0."""
    rng = np.random.default_rng(8)
    case = _rand_case(rng, 1, 64, 3, 4)
    case["dt_bias"] = np.full(3, -60.0)
    got = _call(impl, case)
    want = 2.0 * case["D"][None, None, :] * case["x"] * _silu(case["z"])
    e1 = _rel(got, want)
    case0 = dict(case, D=None)
    got0 = _call(impl, case0)
    e0 = float(np.max(np.abs(got0)))
    return e1 < 1e-14 and e0 < 1e-20, f"rel err {e1:.3e}, |out| with D=0: {e0:.3e}"


def pin_delta_to_inf(impl):
    """P4: dt_bias = +60 makes abar ~ 0, so each state is its own input term.

    out = 2 (Delta_t (C_t . B_t) x_t + D x_t) silu(z_t): pins the Euler input
    term Delta*B*x and the readout.
    """
    rng = np.random.default_rng(9)
    case = _rand_case(rng, 1, 32, 3, 4, a_range=(1.0, 2.0))
    case["dt_bias"] = np.full(3, 60.0)
    dl = _softplus(case["dt"] + 60.0)
    cb = np.sum(case["C"] * case["B"], axis=-1)[:, :, None]
    want = 2.0 * (dl * cb * case["x"] + case["D"][None, None, :] * case["x"]) * _silu(case["z"])
    got = _call(impl, case)
    err = _rel(got, want)
    return err < 1e-12, f"rel err {err:.3e}"


def pin_lti_convolution(impl):
    """P5: constant Delta, B, C turn both scans into causal / anti-causal convolutions.

    Section 3.2 describes the transition kernels as 1D causal and anti-causal
    convolutions; with K_k = sum_n C_n exp(A_n Delta k) Delta B_n (k >= 0),
    y_fwd = K * x (causal) and y_rev = the anti-causal counterpart.
    """
    rng = np.random.default_rng(10)
    nb, L, nd, ns = 1, 120, 2, 3
    case = _rand_case(rng, nb, L, nd, ns)
    case["dt"] = np.broadcast_to(0.5 * rng.standard_normal(nd)[None, None, :], (nb, L, nd)).copy()
    case["B"] = np.broadcast_to(rng.standard_normal(ns)[None, None, :], (nb, L, ns)).copy()
    case["C"] = np.broadcast_to(rng.standard_normal(ns)[None, None, :], (nb, L, ns)).copy()
    case["D"] = None
    want_f = np.zeros((nb, L, nd))
    want_r = np.zeros((nb, L, nd))
    for d in range(nd):
        dl = float(_softplus(case["dt"][0, 0, d] + case["dt_bias"][d]))
        k = np.arange(L)
        K = sum(case["C"][0, 0, n] * np.exp(case["A"][d, n] * dl * k) * dl * case["B"][0, 0, n] for n in range(ns))
        xs = case["x"][0, :, d]
        want_f[0, :, d] = np.convolve(xs, K)[:L]
        want_r[0, :, d] = np.convolve(xs[::-1], K)[:L][::-1]
    ef = _rel(_call(impl, case, fwd=True, rev=False, gate=False), want_f)
    er = _rel(_call(impl, case, fwd=False, rev=True, gate=False), want_r)
    return max(ef, er) < 1e-12, f"rel err fwd {ef:.3e} rev {er:.3e}"


def pin_steady_state(impl):
    """P6: constant inputs give a finite geometric series that tends to ubar B / (1 - abar)."""
    nb, L, nd, ns = 1, 3000, 2, 3
    x = np.full((nb, L, nd), 0.7)
    dt = np.full((nb, L, nd), -1.5)
    B = np.broadcast_to(np.array([0.5, -1.0, 2.0])[None, None, :], (nb, L, ns)).copy()
    C = np.broadcast_to(np.array([1.0, 0.25, -0.5])[None, None, :], (nb, L, ns)).copy()
    A = -np.array([[0.5, 1.0, 3.0], [0.01, 0.2, 1.0]])
    bias = np.array([0.0, -2.0])
    case = dict(x=x, dt=dt, A=A, B=B, C=C, D=None, z=None, dt_bias=bias)
    want_f = np.zeros((nb, L, nd))
    want_r = np.zeros((nb, L, nd))
    t = np.arange(L)
    limit = np.zeros(nd)
    for d in range(nd):
        dl = float(_softplus(-1.5 + bias[d]))
        for n in range(ns):
            a = math.exp(A[d, n] * dl)
            ub = dl * 0.7 * B[0, 0, n]
            want_f[0, :, d] += C[0, 0, n] * ub * (1.0 - a ** (t + 1)) / (1.0 - a)
            want_r[0, :, d] += C[0, 0, n] * ub * (1.0 - a ** (L - t)) / (1.0 - a)
            limit[d] += C[0, 0, n] * ub / (1.0 - a)
    got_f = _call(impl, case, fwd=True, rev=False, gate=False)
    got_r = _call(impl, case, fwd=False, rev=True, gate=False)
    ef = _rel(got_f, want_f)
    er = _rel(got_r, want_r)
    # channel 0 decays fast enough to be at its limit by the end of the sequence
    el = abs(got_f[0, -1, 0] - limit[0]) / abs(limit[0])
    return max(ef, er) < 1e-11 and el < 1e-12, f"rel err fwd {ef:.3e} rev {er:.3e} limit {el:.3e}"


def pin_block_chaining(impl):
    """P7: chaining blocks through the cached forward state reproduces the full forward scan.

    Block-cache decoding (Section 4.3): the forward state is carried across
    blocks exactly; the reverse scan of each block equals the full reverse scan
    of that block's tokens alone.
    """
    rng = np.random.default_rng(11)
    nb, L, nd, ns, G = 2, 48, 3, 4, 8
    case = _rand_case(rng, nb, L, nd, ns)
    full_f = _call(impl, case, fwd=True, rev=False, gate=False)
    h = None
    worst = 0.0
    for b0 in range(0, L, G):
        sl = {k: (case[k][:, b0:b0 + G] if k in ("x", "dt", "z", "B", "C") else case[k]) for k in case}
        out_f, h_next = impl.scan_block(sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["z"], sl["dt_bias"],
                                        h, gate=False, fwd=True, rev=False)
        worst = max(worst, _rel(out_f, full_f[:, b0:b0 + G]))
        out_r, _ = impl.scan_block(sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["z"], sl["dt_bias"],
                                   h, gate=False, fwd=False, rev=True)
        worst = max(worst, _rel(out_r, _call(impl, sl, fwd=False, rev=True, gate=False)))
        # the cached state equals the closed-form forward state at the block end
        want_h = np.zeros((nb, nd, ns))
        dl = _softplus(case["dt"] + case["dt_bias"][None, None, :])
        te = b0 + G - 1
        for s in range(te + 1):
            seg = dl[:, s + 1:te + 1, :].sum(axis=1)  # [nb, nd]
            want_h += (np.exp(case["A"][None] * seg[:, :, None]) * (dl[:, s, :] * case["x"][:, s, :])[:, :, None]
                       * case["B"][:, s, None, :])
        worst = max(worst, _rel(h_next, want_h))
        h = h_next
    return worst < 1e-12, f"max rel err {worst:.3e}"


def pin_linearity(impl):
    """P8: without the gate the output is linear in x for fixed dt, B, C."""
    rng = np.random.default_rng(12)
    c1 = _rand_case(rng, 1, 50, 3, 4)
    c2 = dict(c1, x=rng.standard_normal(c1["x"].shape))
    c3 = dict(c1, x=2.5 * c1["x"] - 0.75 * c2["x"])
    o1 = _call(impl, c1, gate=False)
    o2 = _call(impl, c2, gate=False)
    o3 = _call(impl, c3, gate=False)
    err = _rel(o3, 2.5 * o1 - 0.75 * o2)
    return err < 1e-12, f"rel err {err:.3e}"


def pin_channel_independence(impl):
    """P9: channel d of the output depends only on channel d (B, C are shared)."""
    rng = np.random.default_rng(13)
    case = _rand_case(rng, 2, 30, 6, 4)
    full = _call(impl, case)
    idx = np.array([4, 1])
    sub = dict(case)
    for k in ("x", "dt", "z"):
        sub[k] = case[k][:, :, idx]
    sub["A"] = case["A"][idx]
    sub["D"] = case["D"][idx]
    sub["dt_bias"] = case["dt_bias"][idx]
    part = _call(impl, sub)
    err = float(np.max(np.abs(part - full[:, :, idx])))
    return err == 0.0, f"max abs diff {err:.3e}"


def pin_impulse(impl):
    """P10: an impulse at token s gives C_t diag(prod abar) Delta_s B_s after s and nothing before."""
    rng = np.random.default_rng(14)
    nb, L, nd, ns, s = 1, 300, 2, 4, 120
    case = _rand_case(rng, nb, L, nd, ns, a_range=(0.001, 0.05))
    case["x"] = np.zeros((nb, L, nd))
    case["x"][0, s, :] = 1.0
    case["D"] = None
    dl = _softplus(case["dt"] + case["dt_bias"][None, None, :])[0]
    cum = np.concatenate([np.zeros((1, nd)), np.cumsum(dl, axis=0)])  # cum[k] = sum_{r<k} dl[r]
    want_f = np.zeros((nb, L, nd))
    want_r = np.zeros((nb, L, nd))
    for d in range(nd):
        for t in range(L):
            for n in range(ns):
                base = dl[s, d] * case["B"][0, s, n] * case["C"][0, t, n]
                if t >= s:
                    want_f[0, t, d] += math.exp(case["A"][d, n] * (cum[t + 1, d] - cum[s + 1, d])) * base
                if t <= s:
                    want_r[0, t, d] += math.exp(case["A"][d, n] * (cum[s, d] - cum[t, d])) * base
    ef = _rel(_call(impl, case, fwd=True, rev=False, gate=False), want_f)
    er = _rel(_call(impl, case, fwd=False, rev=True, gate=False), want_r)
    return max(ef, er) < 1e-12, f"rel err fwd {ef:.3e} rev {er:.3e}"


def load_golden(name="hand_example.txt"):
    vals = {}
    env = {"lam": math.log(2.0), "l3": math.log(3.0)}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = np.array(eval(v, {"__builtins__": {}}, env), dtype=np.float64)
    return vals


def pin_golden(impl):
    """Hand-derived three-token example (tests/golden/hand_example.txt)."""
    g = load_golden()
    l3 = math.log(3.0)
    case = dict(
        x=np.array([1.0, 2.0, -1.0]).reshape(1, 3, 1),
        dt=np.zeros((1, 3, 1)),
        A=np.array([[-1.0, -2.0]]),
        B=np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 3, 2),
        C=np.array([[1.0, 1.0], [1.0, 0.0], [0.0, 1.0]]).reshape(1, 3, 2),
        D=np.array([0.5]),
        z=np.array([l3, -l3, 0.0]).reshape(1, 3, 1),
        dt_bias=np.array([0.0]),
    )
    errs = []
    nd = dict(case, D=None)
    errs.append(np.max(np.abs(_call(impl, nd, fwd=True, rev=False, gate=False).ravel() - g["y_fwd"])))
    errs.append(np.max(np.abs(_call(impl, nd, fwd=False, rev=True, gate=False).ravel() - g["y_rev"])))
    errs.append(np.max(np.abs(_call(impl, case).ravel() - g["out"])))
    out_b, h_out = impl.scan_block(case["x"], case["dt"], case["A"], case["B"], case["C"], case["D"], case["z"],
                                   case["dt_bias"], np.ones((1, 1, 2)))
    errs.append(np.max(np.abs(out_b.ravel() - g["block_out"])))
    errs.append(np.max(np.abs(h_out.ravel() - g["block_h_out"])))
    worst = float(max(errs))
    return worst < 1e-14, f"max abs err {worst:.3e}"


def pin_untied(impl):
    """P11: untied directions.  With two different parameter/input sets, out_f equals the forward
    closed form of the first set and out_r the reverse closed form of the second (brute force); with
    both sets equal, out_f + out_r is the tied bidirectional result (the gate distributes over the sum,
    and each direction carries its own D x)."""
    worst = 0.0
    for seed in range(3):
        rng = np.random.default_rng(300 + seed)
        cf = _rand_case(rng, 1 + seed % 2, 6 + 3 * seed, 2, 1 + seed % 3)
        cr = _rand_case(rng, 1 + seed % 2, 6 + 3 * seed, 2, 1 + seed % 3)
        out_f, out_r = impl.scan_fwd_untied(cf, cr)
        worst = max(worst, _rel(out_f, brute_force(cf, fwd=True, rev=False)))
        worst = max(worst, _rel(out_r, brute_force(cr, fwd=False, rev=True)))
        both = _call(impl, cf)
        f2, r2 = impl.scan_fwd_untied(cf, cf)
        worst = max(worst, _rel(f2 + r2, both))
    return worst < 1e-12, f"max rel err {worst:.3e}"


ALL_PINS = [
    pin_brute_force,
    pin_flip,
    pin_delta_to_zero,
    pin_delta_to_inf,
    pin_lti_convolution,
    pin_steady_state,
    pin_block_chaining,
    pin_linearity,
    pin_channel_independence,
    pin_impulse,
    pin_golden,
    pin_untied,
]
