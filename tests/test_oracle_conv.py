"""The fp64 short-convolution oracle against facts it does not define itself, and planted mistakes
that those facts must catch.  CPU only."""
import numpy as np
import pytest

import oracle.conv as oconv
from tests.oracle_pins_conv import ALL_CONV_PINS


@pytest.mark.parametrize("pin", ALL_CONV_PINS, ids=lambda p: p.__name__)
def test_conv_pin(pin):
    ok, detail = pin(oconv)
    assert ok, f"{pin.__name__}: {detail}"


_orig_causal = oconv.conv_causal
_orig_anti = oconv.conv_anticausal
_orig_block = oconv.conv_block


def _causal_taps_reversed(u, w, b=None, cache=None, *, act=True):
    return _orig_causal(u, np.asarray(w)[:, ::-1], b, cache, act=act)


def _causal_no_bias(u, w, b=None, cache=None, *, act=True):
    return _orig_causal(u, w, None, cache, act=act)


def _causal_right_padding(u, w, b=None, cache=None, *, act=True):
    # reads u[t + k] instead of u[t - (K-1) + k]
    u = np.asarray(u, dtype=np.float64)
    K = np.asarray(w).shape[1]
    ext = np.concatenate([u, np.zeros((u.shape[0], K - 1, u.shape[2]))], axis=1)
    out = np.zeros_like(u) if b is None else np.broadcast_to(np.asarray(b, dtype=np.float64), u.shape).copy()
    for t in range(u.shape[1]):
        for k in range(K):
            out[:, t] += np.asarray(w)[None, :, k] * ext[:, t + k]
    return oconv.silu(out) if act else out


def _anti_same_taps_as_causal(u, w, b=None, *, act=True):
    # anti-causal filter with the taps in causal order (w[k] on u[t + k])
    u = np.asarray(u, dtype=np.float64)
    K = np.asarray(w).shape[1]
    ext = np.concatenate([u, np.zeros((u.shape[0], K - 1, u.shape[2]))], axis=1)
    out = np.zeros_like(u) if b is None else np.broadcast_to(np.asarray(b, dtype=np.float64), u.shape).copy()
    for t in range(u.shape[1]):
        for k in range(K):
            out[:, t] += np.asarray(w)[None, :, k] * ext[:, t + k]
    return oconv.silu(out) if act else out


def _block_cache_newest_first(u, w_f, b_f, w_r, b_r, cache=None, *, act=True):
    f, r, c = _orig_block(u, w_f, b_f, w_r, b_r, cache, act=act)
    return f, r, c[:, ::-1, :]


def _block_ignores_cache(u, w_f, b_f, w_r, b_r, cache=None, *, act=True):
    return _orig_block(u, w_f, b_f, w_r, b_r, None, act=act)


MUTANTS = {
    "causal taps reversed": [("conv_causal", _causal_taps_reversed)],
    "causal bias dropped": [("conv_causal", _causal_no_bias)],
    "causal padding on the right": [("conv_causal", _causal_right_padding)],
    "anti-causal taps in causal order": [("conv_anticausal", _anti_same_taps_as_causal)],
    "block cache stored newest first": [("conv_block", _block_cache_newest_first)],
    "block ignores the cache": [("conv_block", _block_ignores_cache)],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_conv_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(oconv, attr, fn)
    failed = []
    for pin in ALL_CONV_PINS:
        try:
            with np.errstate(all="ignore"):
                ok, _ = pin(oconv)
        except (FloatingPointError, OverflowError, ValueError, ZeroDivisionError, IndexError):
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant '{name}'"
