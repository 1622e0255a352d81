"""Plausible mistakes planted in the oracle (on the CPU) must each fail a pin.

Every mutant replaces one helper of oracle.scan for the duration of a test;
the pins of tests/oracle_pins.py are then run against the patched module and
at least one of them has to fail.  This shows the pins would catch a dropped
term, a wrong sign or index, or a transposed operand in the oracle.
"""
import numpy as np
import pytest

import oracle.scan as oscan
from tests.oracle_pins import ALL_PINS


def _fwd_generic(delta, ubar, A, B, C, h0=None, *, shift_in=False, readout_before=False, swap=False, zoh=False,
                 sign=1.0):
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    if swap:
        B, C = C, B
    nb, L, nd = delta.shape
    h = np.zeros((nb, nd, A.shape[1])) if h0 is None else np.asarray(h0, dtype=np.float64).copy()
    y = np.empty((nb, L, nd))
    for t in range(L):
        abar = np.exp(sign * delta[:, t, :, None] * A[None])
        if zoh:
            inp = (abar - 1.0) / A[None] * (ubar[:, t, :] / delta[:, t, :])[:, :, None] * B[:, t, None, :]
        else:
            inp = ubar[:, t, :, None] * B[:, t, None, :]
        if shift_in and t == 0:
            inp = inp * 0.0
        prev = h
        h = abar * h + inp
        y[:, t, :] = np.sum((prev if readout_before else h) * C[:, t, None, :], axis=-1)
    return y, h


def _rev_generic(delta, ubar, A, B, C, g0=None, *, abar_next=False, c_next=False):
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    nb, L, nd = delta.shape
    g = np.zeros((nb, nd, A.shape[1])) if g0 is None else np.asarray(g0, dtype=np.float64).copy()
    y = np.empty((nb, L, nd))
    for t in range(L - 1, -1, -1):
        ta = min(t + 1, L - 1) if abar_next else t
        abar = np.exp(delta[:, ta, :, None] * A[None])
        g = abar * g + ubar[:, t, :, None] * B[:, t, None, :]
        tc = min(t + 1, L - 1) if c_next else t
        y[:, t, :] = np.sum(g * C[:, tc, None, :], axis=-1)
    return y, g


def _discretise_bias_after(x, dt, dt_bias):
    delta = oscan.softplus(dt) + (0.0 if dt_bias is None else np.asarray(dt_bias)[None, None, :])
    return delta, delta * np.asarray(x, dtype=np.float64)


def _discretise_no_bias(x, dt, dt_bias):
    delta = oscan.softplus(dt)
    return delta, delta * np.asarray(x, dtype=np.float64)


def _discretise_exp(x, dt, dt_bias):
    v = np.asarray(dt, dtype=np.float64) + (0.0 if dt_bias is None else np.asarray(dt_bias)[None, None, :])
    delta = np.exp(v)
    return delta, delta * np.asarray(x, dtype=np.float64)


def _combine_single_d(y_f, y_r, x, D, z, gate):
    x = np.asarray(x, dtype=np.float64)
    out = sum(y for y in (y_f, y_r) if y is not None)
    if D is not None:
        out = out + np.asarray(D)[None, None, :] * x
    return out * oscan.silu(z) if gate else out


def _combine_sigmoid(y_f, y_r, x, D, z, gate):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    for y in (y_f, y_r):
        if y is None:
            continue
        out = out + y + (0.0 if D is None else np.asarray(D)[None, None, :] * x)
    return out / (1.0 + np.exp(-np.asarray(z, dtype=np.float64))) if gate else out


def _scan_block_hout_rev(x, dt, A, B, C, D=None, z=None, dt_bias=None, h_in=None, *, gate=True, fwd=True, rev=True):
    delta, ubar = oscan.discretise(x, dt, dt_bias)
    y_f, _ = oscan.forward_scan(delta, ubar, A, B, C, h_in)
    y_r, g = oscan.reverse_scan(delta, ubar, A, B, C)
    return oscan._combine(y_f if fwd else None, y_r if rev else None, x, D, z, gate), g


def _scan_block_rev_from_hin(x, dt, A, B, C, D=None, z=None, dt_bias=None, h_in=None, *, gate=True, fwd=True,
                             rev=True):
    delta, ubar = oscan.discretise(x, dt, dt_bias)
    y_f, h = oscan.forward_scan(delta, ubar, A, B, C, h_in)
    y_r, _ = oscan.reverse_scan(delta, ubar, A, B, C, h_in)
    return oscan._combine(y_f if fwd else None, y_r if rev else None, x, D, z, gate), h


def _p(**kw):
    return lambda *a, **k: _fwd_generic(*a, **k, **kw)


def _r(**kw):
    return lambda *a, **k: _rev_generic(*a, **k, **kw)


def _untied_rev_uses_fwd_params(fwd_set, rev_set, *, gate=True):
    mixed = dict(rev_set)
    for k in ("A", "D", "dt_bias"):
        mixed[k] = fwd_set.get(k)
    return _untied_orig(fwd_set, mixed, gate=gate)


def _untied_shared_gate(fwd_set, rev_set, *, gate=True):
    mixed = dict(rev_set)
    mixed["z"] = fwd_set.get("z")
    return _untied_orig(fwd_set, mixed, gate=gate)


_untied_orig = oscan.scan_fwd_untied


MUTANTS = {
    "reverse uses abar of the next token": [("reverse_scan", _r(abar_next=True))],
    "reverse reads C of the next token": [("reverse_scan", _r(c_next=True))],
    "forward drops the first input": [("forward_scan", _p(shift_in=True))],
    "forward reads out before the update": [("forward_scan", _p(readout_before=True))],
    "B and C swapped in forward": [("forward_scan", _p(swap=True))],
    "zero-order-hold input term": [("forward_scan", _p(zoh=True))],
    "sign of A flipped": [("forward_scan", _p(sign=-1.0))],
    "dt_bias added after softplus": [("discretise", _discretise_bias_after)],
    "dt_bias ignored": [("discretise", _discretise_no_bias)],
    "exp instead of softplus": [("discretise", _discretise_exp)],
    "skip term D counted once": [("_combine", _combine_single_d)],
    "sigmoid gate instead of silu": [("_combine", _combine_sigmoid)],
    "block cache returns the reverse state": [("scan_block", _scan_block_hout_rev)],
    "block reverse starts from the cache": [("scan_block", _scan_block_rev_from_hin)],
    "untied reverse uses the forward parameters": [("scan_fwd_untied", _untied_rev_uses_fwd_params)],
    "untied directions share the forward gate": [("scan_fwd_untied", _untied_shared_gate)],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(oscan, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                ok, _ = pin(oscan)
        except (FloatingPointError, OverflowError, ValueError, ZeroDivisionError):
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant '{name}'"
