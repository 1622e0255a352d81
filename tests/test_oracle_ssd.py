"""The fp64 Mamba-2 (SSD) oracle against facts it does not define itself, and planted
mistakes that those facts must catch.  CPU only."""
import numpy as np
import pytest

import oracle.ssd as ossd
from tests.oracle_pins_ssd import ALL_SSD_PINS


@pytest.mark.parametrize("pin", ALL_SSD_PINS, ids=lambda p: p.__name__)
def test_ssd_pin(pin):
    ok, detail = pin(ossd)
    assert ok, f"{pin.__name__}: {detail}"


def _scan_generic(delta, xh, A, B, C, s0=None, *, reverse=False, abar_next=False, readout_before=False,
                  swap=False, decay_input=False):
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    if swap:
        B, C = C, B
    nb, L, nh, hp = xh.shape
    s = np.zeros((nb, nh, hp, B.shape[-1])) if s0 is None else np.asarray(s0, dtype=np.float64).copy()
    y = np.empty((nb, L, nh, hp))
    order = range(L - 1, -1, -1) if reverse else range(L)
    for t in order:
        ta = min(t + 1, L - 1) if abar_next else t
        abar = np.exp(delta[:, ta, :] * A[None, :])[:, :, None, None]
        inp = (delta[:, t, :, None] * xh[:, t])[:, :, :, None] * B[:, t, None, None, :]
        prev = s
        s = abar * (s + inp) if decay_input else abar * s + inp
        y[:, t] = np.sum((prev if readout_before else s) * C[:, t, None, None, :], axis=-1)
    return y, s


def _fwd(**kw):
    return lambda *a, **k: _scan_generic(*a, **k, **kw)


def _rev(**kw):
    return lambda *a, **k: _scan_generic(*a, **k, reverse=True, **kw)


def _heads_channel_major(x, nheads):
    x = np.asarray(x, dtype=np.float64)
    nb, L, nc = x.shape
    return x.reshape(nb, L, nc // nheads, nheads).transpose(0, 1, 3, 2)


def _discretise_no_bias(dt, dt_bias):
    return ossd.softplus(dt)


def _discretise_heads_reversed(dt, dt_bias):
    return _orig_discretise(dt, dt_bias)[:, :, ::-1]


_orig_discretise = ossd.ssd_discretise
_orig_block = ossd.ssd_scan_block


def _block_reverse_from_cache(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, **kw):
    """The block's reverse recurrence wrongly starts from the cached forward state."""
    if h0 is None or not kw.get("rev", True):
        return _orig_block(x, dt, A, B, C, D, z, dt_bias, h0, **kw)
    out, h_next = _orig_block(x, dt, A, B, C, D, z, dt_bias, h0, **kw)
    nh = len(A)
    xh = ossd._heads(x, nh)
    delta = ossd.ssd_discretise(dt, dt_bias)
    extra = ossd.ssd_reverse_scan(delta, xh, A, B, C, h0)[0] - ossd.ssd_reverse_scan(delta, xh, A, B, C)[0]
    extra = extra.reshape(np.shape(x))
    if kw.get("gate", True):
        extra = extra * ossd.silu(z)
    return out + extra, h_next


def _block_cache_is_reverse_state(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, **kw):
    """The cache handed to the next block is the reverse state after token 0."""
    out, _ = _orig_block(x, dt, A, B, C, D, z, dt_bias, h0, **kw)
    delta = ossd.ssd_discretise(dt, dt_bias)
    return out, ossd.ssd_reverse_scan(delta, ossd._heads(x, len(A)), A, B, C)[1]


MUTANTS = {
    "reverse uses abar of the next token": [("ssd_reverse_scan", _rev(abar_next=True))],
    "forward reads out before the update": [("ssd_forward_scan", _fwd(readout_before=True))],
    "B and C swapped in the reverse scan": [("ssd_reverse_scan", _rev(swap=True))],
    "forward decays the input term too": [("ssd_forward_scan", _fwd(decay_input=True))],
    "channels laid out head-minor": [("_heads", _heads_channel_major)],
    "dt_bias ignored": [("ssd_discretise", _discretise_no_bias)],
    "step sizes of the heads reversed": [("ssd_discretise", _discretise_heads_reversed)],
    "block reverse starts from the cache": [("ssd_scan_block", _block_reverse_from_cache)],
    "block cache is the reverse state": [("ssd_scan_block", _block_cache_is_reverse_state)],
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_ssd_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(ossd, attr, fn)
    failed = []
    for pin in ALL_SSD_PINS:
        try:
            with np.errstate(all="ignore"):
                ok, _ = pin(ossd)
        except (FloatingPointError, OverflowError, ValueError, ZeroDivisionError):
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutant '{name}'"


def test_ssd_skip_term_per_direction():
    """Each direction is a full layer and carries its own D x (Section 3.2, eq. (6) sums two layers)."""
    rng = np.random.default_rng(590)
    from tests.oracle_pins_ssd import call, rand_case
    case = rand_case(rng, 1, 12, 2, 2, 3)
    both = call(ossd, case, gate=False)
    nod = call(ossd, dict(case, D=None), gate=False)
    want = 2.0 * np.repeat(case["D"], 2)[None, None, :] * case["x"]
    np.testing.assert_allclose(both - nod, want, rtol=0, atol=1e-12)
