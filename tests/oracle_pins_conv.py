"""Pins for the fp64 short-convolution oracle: facts fixed by the mathematics, not by the oracle.

Each pin takes an implementation object exposing ``conv_causal``,
``conv_anticausal``, ``conv_bidir`` and ``conv_block`` with the oracle's
signatures and returns ``(ok, detail)``.  Expected values come from
np.convolve, from an impulse response written out by hand, from a
hand-derived fixture (tests/golden/conv_hand_example.txt) and from the
time-reversal and block-chaining identities.

Table and section numbers refer to "DiffuMamba: High-Throughput Diffusion LMs
with Mamba Backbone" (arXiv v4).
"""
from __future__ import annotations

import os

import numpy as np

from tests.oracle_pins import GOLDEN, _rel, _silu


def rand_conv(rng, nb, L, nc, K=4):
    return dict(u=rng.standard_normal((nb, L, nc)), w_f=rng.standard_normal((nc, K)), b_f=rng.standard_normal(nc),
                w_r=rng.standard_normal((nc, K)), b_r=rng.standard_normal(nc))


def pin_conv_np_convolve(impl):
    """V1: each channel's pre-activation is np.convolve with the reversed filter (causal) and its
    time-reversed counterpart (anti-causal); the activation is u * sigmoid(u)."""
    rng = np.random.default_rng(700)
    cs = rand_conv(rng, 2, 37, 5)
    u = cs["u"]
    want_f = np.zeros_like(u)
    want_r = np.zeros_like(u)
    L = u.shape[1]
    for b in range(u.shape[0]):
        for c in range(u.shape[2]):
            want_f[b, :, c] = np.convolve(u[b, :, c], cs["w_f"][c, ::-1])[:L] + cs["b_f"][c]
            want_r[b, :, c] = np.convolve(u[b, ::-1, c], cs["w_r"][c, ::-1])[:L][::-1] + cs["b_r"][c]
    f, r = impl.conv_bidir(u, cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"])
    err = max(_rel(f, _silu(want_f)), _rel(r, _silu(want_r)))
    fp, rp = impl.conv_bidir(u, cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"], act=False)
    err = max(err, _rel(fp, want_f), _rel(rp, want_r))
    return err < 1e-13, f"rel err {err:.3e}"


def pin_conv_flip(impl):
    """V2: the anti-causal filter is the causal one run on the flipped sequence."""
    rng = np.random.default_rng(701)
    cs = rand_conv(rng, 2, 29, 3)
    r = impl.conv_anticausal(cs["u"], cs["w_r"], cs["b_r"])
    f = impl.conv_causal(cs["u"][:, ::-1, :], cs["w_r"], cs["b_r"])[:, ::-1, :]
    err = _rel(r, f)
    return err < 1e-14, f"rel err {err:.3e}"


def pin_conv_impulse(impl):
    """V3: a unit impulse at token s gives the filter taps: fwd_pre[s + m] = w_f[K-1-m] and
    rev_pre[s - m] = w_r[K-1-m] for m = 0..K-1, zero elsewhere."""
    nc, L, s, K = 3, 20, 9, 4
    rng = np.random.default_rng(702)
    w_f = rng.standard_normal((nc, K))
    w_r = rng.standard_normal((nc, K))
    u = np.zeros((1, L, nc))
    u[0, s, :] = 1.0
    f, r = impl.conv_bidir(u, w_f, None, w_r, None, act=False)
    want_f = np.zeros((1, L, nc))
    want_r = np.zeros((1, L, nc))
    for m in range(K):
        want_f[0, s + m, :] = w_f[:, K - 1 - m]
        want_r[0, s - m, :] = w_r[:, K - 1 - m]
    err = max(float(np.max(np.abs(f - want_f))), float(np.max(np.abs(r - want_r))))
    return err == 0.0, f"max abs err {err:.3e}"


def pin_conv_block_chaining(impl):
    """V4: blocks chained through the cache reproduce the full causal filter, each block's reverse
    filter is the anti-causal filter of that block alone, and the cache is the last K-1 tokens."""
    rng = np.random.default_rng(703)
    cs = rand_conv(rng, 2, 50, 4)
    u = cs["u"]
    full_f = impl.conv_causal(u, cs["w_f"], cs["b_f"])
    cache = None
    worst = 0.0
    for b0, G in ((0, 7), (7, 1), (8, 2), (10, 16), (26, 24)):
        blk = u[:, b0:b0 + G]
        f, r, cache_next = impl.conv_block(blk, cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"], cache)
        worst = max(worst, _rel(f, full_f[:, b0:b0 + G]))
        worst = max(worst, _rel(r, impl.conv_anticausal(blk, cs["w_r"], cs["b_r"])))
        lo = b0 + G - 3
        want_cache = np.concatenate([np.zeros((2, 3, 4)), u], axis=1)[:, lo + 3:lo + 6]
        worst = max(worst, float(np.max(np.abs(cache_next - want_cache))))
        cache = cache_next
    return worst < 1e-14, f"max err {worst:.3e}"


def load_conv_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "conv_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = np.array(eval(v, {"__builtins__": {}}, {}), dtype=np.float64)
    return vals


def pin_conv_golden(impl):
    """Hand-derived example (tests/golden/conv_hand_example.txt)."""
    g = load_conv_golden()
    w = np.array([[1.0, 10.0, 100.0, 1000.0]])
    u = np.array([1.0, 2.0, 3.0]).reshape(1, 3, 1)
    f, r = impl.conv_bidir(u, w, None, w, None, act=False)
    errs = [np.abs(f.ravel() - g["fwd_pre"]).max(), np.abs(r.ravel() - g["rev_pre"]).max()]
    cache = np.array([4.0, 5.0, 6.0]).reshape(1, 3, 1)
    bf, _, co = impl.conv_block(u, w, None, w, None, cache, act=False)
    errs += [np.abs(bf.ravel() - g["block_fwd_pre"]).max(), np.abs(co.ravel() - g["block_cache_out"]).max()]
    one = np.array([7.0]).reshape(1, 1, 1)
    of, orr, oc = impl.conv_block(one, w, None, w, None, cache, act=False)
    errs += [np.abs(of.ravel() - g["one_fwd_pre"]).max(), np.abs(orr.ravel() - g["one_rev_pre"]).max(),
             np.abs(oc.ravel() - g["one_cache_out"]).max()]
    worst = float(max(errs))
    return worst == 0.0, f"max abs err {worst:.3e}"


ALL_CONV_PINS = [pin_conv_np_convolve, pin_conv_flip, pin_conv_impulse, pin_conv_block_chaining, pin_conv_golden]
