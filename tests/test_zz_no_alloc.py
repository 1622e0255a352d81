"""The allocation-free entry point (bimamba_scan_fwd_noalloc) against bimamba_scan_fwd, through the C ABI.

Both run the same kernels on the same inputs, one with a caller workspace and one with the library's fixed
scratch array, so their outputs must be equal bit for bit.  Two calls in a row, the second with a smaller
problem than the first (the scratch array keeps the first call's contents), and a third that is larger
again; then a problem past the scratch size is rejected.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import say, upload

pytestmark = pytest.mark.gpu


def _inputs(batch, L, D, N, io, seed):
    A, Dv, bias = I.make_params(D, N, a_jitter=0.2 if seed % 2 else 0.0)
    act = I.make_activations(batch, L, D, N, io, seed=seed)
    act.update(A=A, D=Dv, dt_bias=bias)
    return upload(act, io)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()
    yield


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_fwd, bimamba_scan_fwd_noalloc

    cases = [(2, 3000, 256, 16, "bf16", 1, 0), (1, 700, 128, 16, "f32", 2, 0), (1, 2048, 4096, 16, "bf16", 3, 0),
             (1, 333, 64, 5, "f32", 5, 1)]
    for batch, L, D, N, io, seed, flags in cases:
        say(f"noalloc: batch {batch} L {L} d_inner {D} N {N} {io} flags {flags}")
        dev = _inputs(batch, L, D, N, io, seed)
        z = None if flags & 1 else dev["z"]
        args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], z, dev["dt_bias"])
        want = bimamba_scan_fwd(*args, flags=flags)
        got = bimamba_scan_fwd_noalloc(*args, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"noalloc differs from the workspace call at {batch}x{L}x{D}x{N} {io}"


def test_noalloc_rejects_problems_past_the_scratch():
    import torch

    from bidirectional_mamba_selective_amd import BimambaError, bimamba_scan_fwd_noalloc
    from bidirectional_mamba_selective_amd._lib import BIMAMBA_ERR_SCRATCH_TOO_SMALL

    dev = _inputs(1, 16384, 4096, 16, "bf16", 7)
    with pytest.raises(BimambaError) as e:
        bimamba_scan_fwd_noalloc(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                                 dev["dt_bias"])
    assert e.value.status == BIMAMBA_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
