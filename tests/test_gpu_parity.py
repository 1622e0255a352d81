"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Bars: normwise relative error <= 2e-2 with bf16 I/O and <= 1e-4 with fp32 I/O
on the whole output (and, where stated, on the SSM-only output obtained with
D = NULL and the gate off, which a broken carry cannot hide behind).  Full-size
workloads are checked on a channel subset: output channel d depends only on
channel d and the shared B, C, so the oracle on a subset is exact for it.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import oracle_fwd, rel_err, run_fwd, say, to_host64, tol_for, upload

pytestmark = pytest.mark.gpu

NO_GATE, FWD_ONLY, REV_ONLY = 1, 2, 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()  # raises if libbimamba.so is missing
    yield


def case(batch, L, D, N, io, seed=1, a_jitter=0.0):
    A, Dv, bias = I.make_params(D, N, a_jitter=a_jitter)
    act = I.make_activations(batch, L, D, N, io, seed=seed)
    act.update(A=A, D=Dv, dt_bias=bias)
    return act


VARIANTS = [
    ("full", 0, dict()),
    ("ssm_only", NO_GATE, dict(use_D=False)),
    ("fwd_only", FWD_ONLY, dict()),
    ("rev_only_nogate", REV_ONLY | NO_GATE, dict()),
    ("no_bias", 0, dict(use_bias=False)),
]


def check_variants(inp, io, variants=VARIANTS, chan=None, tag=""):
    dev = upload(inp, io)
    for name, flags, kw in variants:
        say(f"{tag} variant {name} flags={flags}")
        out = to_host64(run_fwd(dev, flags=flags, use_D=kw.get("use_D", True), use_bias=kw.get("use_bias", True),
                                use_z=not (flags & NO_GATE)))
        want = oracle_fwd(inp, chan=chan, gate=not (flags & NO_GATE), fwd=not (flags & REV_ONLY),
                          rev=not (flags & FWD_ONLY), use_D=kw.get("use_D", True),
                          use_bias=kw.get("use_bias", True))
        got = out if chan is None else out[:, :, chan]
        err = rel_err(got, want)
        say(f"{tag} {name}: rel err {err:.3e}")
        assert np.all(np.isfinite(got)), f"{tag} {name}: non-finite output"
        assert err <= tol_for(io), f"{tag} {name}: rel err {err:.3e} > {tol_for(io)}"


def test_tiny_fp32_workload():
    """batch 1, L 256, d_inner 64, d_state 16, fp32 I/O."""
    w = I.WORKLOADS["tiny_fp32"]
    check_variants(case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype), w.io_dtype, tag="tiny_fp32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("a_jitter", [0.0, 0.2])
def test_ragged_multichunk(io, a_jitter):
    """Many chunks, a ragged last chunk and a ragged last sub-chunk, batch 2; A with (jitter 0) and without
    (jitter 0.2) the per-channel geometric structure."""
    check_variants(case(2, 1000, 128, 16, io, a_jitter=a_jitter), io, tag=f"ragged_{io}_j{a_jitter}")


@pytest.mark.parametrize("N", [1, 3, 4, 5, 8, 12, 16])
@pytest.mark.parametrize("a_jitter", [0.0, 0.2])
def test_state_sizes(N, a_jitter):
    check_variants(case(1, 333, 64, N, "f32", seed=N, a_jitter=a_jitter), "f32", variants=VARIANTS[:2],
                   tag=f"N{N}_j{a_jitter}")


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 31, 33, 4097])
def test_lengths(L):
    check_variants(case(1, L, 64, 16, "f32", seed=L), "f32", variants=VARIANTS[:2], tag=f"L{L}")


def test_general_A_matrix():
    """A without the per-channel geometric structure of the default init."""
    check_variants(case(1, 700, 192, 16, "f32", a_jitter=0.3), "f32", variants=VARIANTS[:2], tag="jitterA")


def test_mixed_A_rows():
    """Geometric rows in some wavefronts and general rows in others (and one general row inside an otherwise
    geometric wavefront): each wavefront picks its own path."""
    inp = case(1, 900, 256, 16, "f32")
    A = inp["A"].copy()
    A[64:128] *= np.float32(1.0) + np.float32(0.05) * np.linspace(-1, 1, 16, dtype=np.float32)[None, :]
    A[200, 7] *= np.float32(1.001)
    inp["A"] = A
    check_variants(inp, "f32", variants=VARIANTS[:2], tag="mixedA")


def test_geometric_rows_other_than_default():
    """A[d, n] = (n + 1) * a_d with a per-channel a_d != -1 (still geometric)."""
    inp = case(1, 900, 128, 16, "f32")
    a = -np.exp(np.random.default_rng(3).uniform(-1.0, 1.0, size=128)).astype(np.float32)
    inp["A"] = (a[:, None] * np.arange(1, 17, dtype=np.float32)[None, :]).astype(np.float32)
    check_variants(inp, "f32", variants=VARIANTS[:2], tag="geoA")


@pytest.mark.parametrize("a_jitter", [0.0, 0.2])
def test_impulse_crosses_chunks(a_jitter):
    """An impulse in one channel set: every other output is carry-only (both directions)."""
    inp = case(1, 4000, 64, 16, "f32", a_jitter=a_jitter)
    inp["x"] = np.zeros_like(inp["x"])
    inp["x"][0, 1234, :] = 1.0
    inp["dt_bias"] = np.full_like(inp["dt_bias"], -6.0)  # delta ~ 2.5e-3: memory of thousands of tokens
    dev = upload(inp, "f32")
    out = to_host64(run_fwd(dev, flags=NO_GATE, use_D=False, use_z=False))
    want = oracle_fwd(inp, gate=False, use_D=False)
    err = rel_err(out, want)
    far = rel_err(out[:, :200], want[:, :200]) + rel_err(out[:, 3800:], want[:, 3800:])
    say(f"impulse: rel err {err:.3e}, far-field {far:.3e}")
    assert err <= 1e-4 and far <= 2e-4


def test_deterministic():
    inp = case(2, 1500, 256, 16, "bf16")
    dev = upload(inp, "bf16")
    a = run_fwd(dev)
    b = run_fwd(dev)
    import torch

    assert torch.equal(a, b), "two identical runs differ"


def test_layer_2k_workload():
    """batch 1, L 2048, d_inner 4096, d_state 16, bf16 I/O: full oracle, all variants."""
    w = I.WORKLOADS["layer_2k_bf16"]
    inp = case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype)
    chan = np.arange(0, w.d_inner, 4)  # 1024 channels keep the oracle fast
    check_variants(inp, w.io_dtype, variants=VARIANTS[:4], chan=chan, tag="layer_2k")


@pytest.mark.parametrize("a_jitter", [0.0, 0.2])
def test_layer_2k_fp32_ssm_only(a_jitter):
    """Same shape with fp32 I/O: the SSM-only part at the tight fp32 bar."""
    inp = case(1, 2048, 4096, 16, "f32", a_jitter=a_jitter)
    chan = np.arange(3, 4096, 16)
    check_variants(inp, "f32", variants=VARIANTS[1:2], chan=chan, tag="layer_2k_f32")


def test_long_64k_workload():
    """batch 1, L 65536, d_inner 4096, d_state 16, bf16: the benchmarked launch, channel-subset oracle."""
    w = I.WORKLOADS["long_64k_bf16"]
    say("long_64k: generating inputs")
    inp = case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype)
    chan = np.concatenate([np.arange(0, 64, 7), np.arange(2000, 2064, 9), np.arange(4032, 4096, 5)])
    check_variants(inp, w.io_dtype, variants=VARIANTS[:2], chan=chan, tag="long_64k")


def test_long_64k_general_A():
    """The L = 65536 launch with A off the geometric structure (general exponential path)."""
    w = I.WORKLOADS["long_64k_bf16"]
    inp = case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, a_jitter=0.2)
    chan = np.arange(17, w.d_inner, 211)
    check_variants(inp, w.io_dtype, variants=VARIANTS[1:2], chan=chan, tag="long_64k_jitterA")


@pytest.mark.parametrize("shift", [-60.0, -20.0, 20.0, 60.0])
@pytest.mark.parametrize("a_jitter", [0.0, 0.2])
def test_delta_limits(shift, a_jitter):
    """dt_bias shifted far down (delta -> 0: abar -> 1 and almost no input; at -60 the output is
    2 D x SiLU(z) to within e^-60) and far up (delta ~ dt + bias: abar -> 0, the state is the
    current input, powers of abar underflow) in fp32, both A paths, against the oracle."""
    inp = case(2, 300, 128, 16, "f32", seed=int(abs(shift)) + 3, a_jitter=a_jitter)
    inp["dt_bias"] = (inp["dt_bias"] + np.float32(shift)).astype(np.float32)
    check_variants(inp, "f32", variants=VARIANTS[:2], tag=f"delta_shift{shift:+.0f}")
