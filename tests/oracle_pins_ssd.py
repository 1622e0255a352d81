"""Pins for the fp64 Mamba-2 (SSD) oracle: facts fixed by the mathematics, not by the oracle.

Each pin takes an implementation object exposing ``ssd_scan_fwd`` (and, for
the state pin, ``ssd_forward_scan`` / ``ssd_reverse_scan``) with the oracle's
signatures and returns ``(ok, detail)``.  The expected values come from
closed forms written out here with their own formulas (logaddexp softplus,
a plain-division SiLU, explicit segment sums), from np.convolve, and from the
separately pinned per-channel S6 oracle with its transition tied across the
state index.

Section and table numbers refer to "DiffuMamba: High-Throughput Diffusion LMs
with Mamba Backbone" (arXiv v4).
"""
from __future__ import annotations

import math

import numpy as np

from tests.oracle_pins import _rel, _silu, _softplus


def rand_case(rng, nb, L, nh, hp, ns, a_range=(0.5, 4.0)):
    """Random SSD problem in the oracle's layout (x, z: [nb, L, nh*hp]; dt: [nb, L, nh])."""
    nc = nh * hp
    return dict(
        x=rng.standard_normal((nb, L, nc)),
        dt=0.5 * rng.standard_normal((nb, L, nh)),
        z=rng.standard_normal((nb, L, nc)),
        B=rng.standard_normal((nb, L, ns)),
        C=rng.standard_normal((nb, L, ns)),
        A=-rng.uniform(*a_range, size=nh),
        D=rng.standard_normal(nh),
        dt_bias=rng.uniform(-3.0, 0.5, size=nh),
    )


def call(impl, case, **kw):
    return impl.ssd_scan_fwd(case["x"], case["dt"], case["A"], case["B"], case["C"], case.get("D"), case.get("z"),
                             case.get("dt_bias"), **kw)


def brute_force(case, fwd=True, rev=True, gate=True):
    """Unrolled closed form by explicit loops (the masked "attention" form of a scalar-decay SSM).

    y_fwd[t, h, p] = sum_{s<=t} (C_t . B_s) exp(A_h sum_{r=s+1..t} Delta_r,h) Delta_s,h x_s,h,p
    y_rev[t, h, p] = sum_{s>=t} (C_t . B_s) exp(A_h sum_{r=t..s-1} Delta_r,h) Delta_s,h x_s,h,p
    each direction plus D_h x_t,h,p, summed, times silu(z).
    """
    x, dt, B, C = (np.asarray(case[k], dtype=np.float64) for k in ("x", "dt", "B", "C"))
    A = np.asarray(case["A"], dtype=np.float64)
    nb, L, nc = x.shape
    nh = A.shape[0]
    hp = nc // nh
    bias = case.get("dt_bias")
    dl = _softplus(dt + (0.0 if bias is None else np.asarray(bias)[None, None, :]))
    Dv = case.get("D")
    out = np.zeros((nb, L, nc))
    for b in range(nb):
        for h in range(nh):
            for p in range(hp):
                c = h * hp + p
                for t in range(L):
                    acc = 0.0
                    if fwd:
                        for s in range(t + 1):
                            cb = float(np.dot(C[b, t], B[b, s]))
                            acc += cb * math.exp(A[h] * dl[b, s + 1:t + 1, h].sum()) * dl[b, s, h] * x[b, s, c]
                        if Dv is not None:
                            acc += Dv[h] * x[b, t, c]
                    if rev:
                        for s in range(t, L):
                            cb = float(np.dot(C[b, t], B[b, s]))
                            acc += cb * math.exp(A[h] * dl[b, t:s, h].sum()) * dl[b, s, h] * x[b, s, c]
                        if Dv is not None:
                            acc += Dv[h] * x[b, t, c]
                    out[b, t, c] = acc
    if gate:
        out = out * _silu(case["z"])
    return out


def pin_ssd_brute_force(impl, seeds=range(5)):
    """S1: the recurrences equal their unrolled closed form (tiny sizes, several seeds)."""
    worst = 0.0
    for seed in seeds:
        rng = np.random.default_rng(500 + seed)
        case = rand_case(rng, 1 + seed % 2, 4 + 2 * seed, 1 + seed % 3, 1 + seed % 3, 1 + seed % 4)
        for fwd, rev, gate in ((True, True, True), (True, False, False), (False, True, False)):
            worst = max(worst, _rel(call(impl, case, fwd=fwd, rev=rev, gate=gate),
                                    brute_force(case, fwd=fwd, rev=rev, gate=gate)))
    return worst < 1e-12, f"max rel err {worst:.3e}"


def pin_ssd_is_tied_s6(impl):
    """S2: a head of the SSD scan is the per-channel S6 scan with A[c, n] = A[h] for every n,
    Delta shared by the head's channels and D, dt_bias repeated per channel (channel c = h * hp + p).

    The S6 oracle is pinned on its own (closed form, flip, limits, convolution, golden example).
    """
    import oracle.scan as s6
    rng = np.random.default_rng(520)
    nb, L, nh, hp, ns = 2, 37, 3, 4, 5
    case = rand_case(rng, nb, L, nh, hp, ns)
    head_of = np.repeat(np.arange(nh), hp)
    A6 = np.repeat(case["A"][head_of][:, None], ns, axis=1)
    worst = 0.0
    for fwd, rev, gate in ((True, True, True), (True, False, True), (False, True, False)):
        want = s6.scan_fwd(case["x"], case["dt"][:, :, head_of], A6, case["B"], case["C"], case["D"][head_of],
                           case["z"], case["dt_bias"][head_of], gate=gate, fwd=fwd, rev=rev)
        worst = max(worst, _rel(call(impl, case, fwd=fwd, rev=rev, gate=gate), want))
    return worst < 1e-13, f"max rel err {worst:.3e}"


def pin_ssd_flip(impl):
    """S3: the reverse scan is the forward scan of the time-reversed input."""
    rng = np.random.default_rng(530)
    case = rand_case(rng, 2, 41, 2, 3, 4)
    flipped = dict(case)
    for k in ("x", "dt", "z", "B", "C"):
        flipped[k] = case[k][:, ::-1, :].copy()
    rev = call(impl, case, fwd=False, rev=True, gate=False)
    fwd_of_flip = call(impl, flipped, fwd=True, rev=False, gate=False)[:, ::-1, :]
    err = _rel(rev, fwd_of_flip)
    return err < 1e-13, f"rel err {err:.3e}"


def pin_ssd_delta_to_zero(impl):
    """S4: dt_bias = -60 makes Delta ~ 1e-26, so out = 2 D_h x silu(z), and ~0 with D = 0."""
    rng = np.random.default_rng(540)
    case = rand_case(rng, 1, 50, 3, 2, 4)
    case["dt_bias"] = np.full(3, -60.0)
    want = 2.0 * np.repeat(case["D"], 2)[None, None, :] * case["x"] * _silu(case["z"])
    e1 = _rel(call(impl, case), want)
    e0 = float(np.max(np.abs(call(impl, dict(case, D=None)))))
    return e1 < 1e-14 and e0 < 1e-20, f"rel err {e1:.3e}, |out| with D=0: {e0:.3e}"


def pin_ssd_lti_convolution(impl):
    """S5: constant Delta, B, C make each direction a causal / anti-causal convolution per channel
    with kernel K_k = (C . B) exp(A_h Delta_h k) Delta_h, k >= 0 (Section 3.2's convolution view)."""
    rng = np.random.default_rng(550)
    nb, L, nh, hp, ns = 1, 90, 2, 3, 4
    case = rand_case(rng, nb, L, nh, hp, ns)
    case["dt"] = np.broadcast_to(0.5 * rng.standard_normal(nh)[None, None, :], (nb, L, nh)).copy()
    case["B"] = np.broadcast_to(rng.standard_normal(ns)[None, None, :], (nb, L, ns)).copy()
    case["C"] = np.broadcast_to(rng.standard_normal(ns)[None, None, :], (nb, L, ns)).copy()
    case["D"] = None
    cb = float(np.dot(case["B"][0, 0], case["C"][0, 0]))
    want_f = np.zeros((nb, L, nh * hp))
    want_r = np.zeros((nb, L, nh * hp))
    k = np.arange(L)
    for h in range(nh):
        dl = float(_softplus(case["dt"][0, 0, h] + case["dt_bias"][h]))
        K = cb * np.exp(case["A"][h] * dl * k) * dl
        for p in range(hp):
            xs = case["x"][0, :, h * hp + p]
            want_f[0, :, h * hp + p] = np.convolve(xs, K)[:L]
            want_r[0, :, h * hp + p] = np.convolve(xs[::-1], K)[:L][::-1]
    ef = _rel(call(impl, case, fwd=True, rev=False, gate=False), want_f)
    er = _rel(call(impl, case, fwd=False, rev=True, gate=False), want_r)
    return max(ef, er) < 1e-12, f"rel err fwd {ef:.3e} rev {er:.3e}"


def pin_ssd_head_independence(impl):
    """S6: head h of the output depends only on head h's channels, dt, A, D and bias."""
    rng = np.random.default_rng(560)
    nh, hp = 5, 3
    case = rand_case(rng, 2, 23, nh, hp, 4)
    full = call(impl, case)
    heads = [3, 0]
    cols = np.concatenate([np.arange(h * hp, (h + 1) * hp) for h in heads])
    sub = dict(case)
    for k in ("x", "z"):
        sub[k] = case[k][:, :, cols]
    sub["dt"] = case["dt"][:, :, heads]
    for k in ("A", "D", "dt_bias"):
        sub[k] = case[k][heads]
    err = float(np.max(np.abs(call(impl, sub) - full[:, :, cols])))
    return err == 0.0, f"max abs diff {err:.3e}"


def pin_ssd_states(impl):
    """S7: the final states equal their closed forms
    H_L = sum_s exp(A_h sum_{r>s} Delta_r) Delta_s x_s (outer) B_s and
    G_0 = sum_s exp(A_h sum_{r<s} Delta_r) Delta_s x_s (outer) B_s."""
    rng = np.random.default_rng(570)
    nb, L, nh, hp, ns = 2, 29, 2, 3, 4
    case = rand_case(rng, nb, L, nh, hp, ns)
    dl = _softplus(case["dt"] + case["dt_bias"][None, None, :])
    xh = case["x"].reshape(nb, L, nh, hp)
    want_h = np.zeros((nb, nh, hp, ns))
    want_g = np.zeros((nb, nh, hp, ns))
    for s in range(L):
        after = dl[:, s + 1:, :].sum(axis=1)
        before = dl[:, :s, :].sum(axis=1)
        term = (dl[:, s, :, None] * xh[:, s])[:, :, :, None] * case["B"][:, s, None, None, :]
        want_h += np.exp(case["A"][None] * after)[:, :, None, None] * term
        want_g += np.exp(case["A"][None] * before)[:, :, None, None] * term
    delta = impl.ssd_discretise(case["dt"], case["dt_bias"])
    _, h = impl.ssd_forward_scan(delta, xh, case["A"], case["B"], case["C"])
    _, g = impl.ssd_reverse_scan(delta, xh, case["A"], case["B"], case["C"])
    err = max(_rel(h, want_h), _rel(g, want_g))
    return err < 1e-12, f"rel err {err:.3e}"


def pin_ssd_linearity(impl):
    """S8: without the gate the output is linear in x for fixed dt, B, C."""
    rng = np.random.default_rng(580)
    c1 = rand_case(rng, 1, 33, 2, 3, 4)
    c2 = dict(c1, x=rng.standard_normal(c1["x"].shape))
    c3 = dict(c1, x=1.5 * c1["x"] - 2.0 * c2["x"])
    err = _rel(call(impl, c3, gate=False), 1.5 * call(impl, c1, gate=False) - 2.0 * call(impl, c2, gate=False))
    return err < 1e-12, f"rel err {err:.3e}"


def pin_ssd_block_chaining(impl):
    """S9: block-cache decoding (Section 4.3, block-cache paragraph).  Chaining blocks through the cached
    forward state reproduces the full forward scan; each block's reverse output is the reverse scan of
    that block alone; the cache equals the closed-form forward state at the block's end (whatever
    directions the output keeps)."""
    rng = np.random.default_rng(590)
    nb, L, nh, hp, ns, G = 2, 40, 2, 3, 4, 8
    case = rand_case(rng, nb, L, nh, hp, ns)
    full_f = call(impl, case, fwd=True, rev=False, gate=False)
    dl = _softplus(case["dt"] + case["dt_bias"][None, None, :])
    xh = case["x"].reshape(nb, L, nh, hp)
    h = None
    worst = 0.0
    for b0 in range(0, L, G):
        sl = {k: (case[k][:, b0:b0 + G] if k in ("x", "dt", "z", "B", "C") else case[k]) for k in case}
        args = [sl[k] for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")]
        out_f, h_next = impl.ssd_scan_block(*args, h, gate=False, fwd=True, rev=False)
        worst = max(worst, _rel(out_f, full_f[:, b0:b0 + G]))
        out_r, h_r = impl.ssd_scan_block(*args, h, gate=False, fwd=False, rev=True)
        worst = max(worst, _rel(out_r, call(impl, sl, fwd=False, rev=True, gate=False)))
        worst = max(worst, _rel(h_r, h_next))
        te = b0 + G - 1
        want = np.zeros((nb, nh, hp, ns))
        for s_ in range(te + 1):
            seg = dl[:, s_ + 1:te + 1, :].sum(axis=1)  # [nb, nh]
            term = (dl[:, s_, :, None] * xh[:, s_])[:, :, :, None] * case["B"][:, s_, None, None, :]
            want += np.exp(case["A"][None] * seg)[:, :, None, None] * term
        worst = max(worst, _rel(h_next, want))
        h = h_next
    return worst < 1e-12, f"max rel err {worst:.3e}"


ALL_SSD_PINS = [
    pin_ssd_brute_force,
    pin_ssd_is_tied_s6,
    pin_ssd_flip,
    pin_ssd_delta_to_zero,
    pin_ssd_lti_convolution,
    pin_ssd_head_independence,
    pin_ssd_states,
    pin_ssd_linearity,
    pin_ssd_block_chaining,
]
