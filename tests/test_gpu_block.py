"""Block-cache variant and multi-call workloads against the fp64 oracle.

Block decoding (Section 4.3, block-cache paragraph): the forward state is
carried across blocks, the reverse scan stays inside the active block.  The
cached state is fp32 and is checked at the tight fp32 bar at every block
boundary.
"""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import f32_dev, oracle_fwd, rel_err, say, to_dev, to_host64, tol_for, upload

pytestmark = pytest.mark.gpu

NO_GATE, FWD_ONLY, REV_ONLY = 1, 2, 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()
    yield


def _case(batch, L, D, N, io, seed=1):
    A, Dv, bias = I.make_params(D, N)
    act = I.make_activations(batch, L, D, N, io, seed=seed)
    act.update(A=A, D=Dv, dt_bias=bias)
    return act


def _block_call(dev, sl, h_in, h_out, flags=0):
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_block

    out = bimamba_scan_block(sl["x"], sl["dt"], dev["A"], sl["B"], sl["C"], dev["D"],
                             None if flags & NO_GATE else sl["z"], dev["dt_bias"], h_in=h_in, h_out=h_out,
                             flags=flags)
    torch.cuda.synchronize()
    return out


def _slice(dev, b0, b1):
    return {k: dev[k][:, b0:b1].contiguous() for k in ("x", "dt", "z", "B", "C")}


@pytest.mark.parametrize("G", [1, 5, 16, 32, 64, 100, 128, 129, 200])
@pytest.mark.parametrize("flags", [0, NO_GATE, FWD_ONLY, REV_ONLY | NO_GATE])
def test_block_small(G, flags):
    """One block with a random cached state; out and h_out against oracle.scan_block (fp32 I/O)."""
    import torch

    inp = _case(2, G, 128, 16, "f32", seed=G)
    rng = np.random.default_rng(G)
    h0 = rng.standard_normal((2, 128, 16)).astype(np.float32)
    dev = upload(inp, "f32")
    h_in = f32_dev(h0)
    h_out = torch.empty_like(h_in)
    out = to_host64(_block_call(dev, dev, h_in, h_out, flags))
    want, want_h = oracle.scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                     None if flags & NO_GATE else inp["z"], inp["dt_bias"], h0,
                                     gate=not (flags & NO_GATE), fwd=not (flags & REV_ONLY),
                                     rev=not (flags & FWD_ONLY))
    e_out = rel_err(out, want)
    e_h = rel_err(to_host64(h_out), want_h)
    say(f"block G={G} flags={flags}: out {e_out:.3e} h_out {e_h:.3e}")
    assert e_out <= 1e-4 and e_h <= 1e-5


@pytest.mark.parametrize("N", [1, 5, 16])
@pytest.mark.parametrize("G", [7, 33, 100])
@pytest.mark.parametrize("jitter", [0.0, 0.2])
def test_block_state_counts(N, G, jitter):
    """Blocks short enough for the single-kernel path, with state counts that leave the last wavefront
    of a workgroup partly or wholly idle, general and geometric A, batch 2, cache updated in place."""
    import torch

    A, Dv, bias = I.make_params(128, N, a_jitter=jitter)
    inp = I.make_activations(2, G, 128, N, "f32", seed=3 + G + N)
    inp.update(A=A, D=Dv, dt_bias=bias)
    dev = upload(inp, "f32")
    rng = np.random.default_rng(N * 100 + G)
    h0 = rng.standard_normal((2, 128, N)).astype(np.float32)
    h = f32_dev(h0)
    out = to_host64(_block_call(dev, dev, h, h))
    want, want_h = oracle.scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                     inp["dt_bias"], h0)
    e_out, e_h = rel_err(out, want), rel_err(to_host64(h), want_h)
    say(f"block N={N} G={G} jitter={jitter}: out {e_out:.3e} h_out {e_h:.3e}")
    assert e_out <= 1e-4 and e_h <= 1e-5


@pytest.mark.parametrize("G", [32, 64, 128, 200])
def test_block_reruns_then_commit(G):
    """Block-diffusion decoding: the active block is denoised k = 4 times from the same cached state
    (fresh x, z each time; the cache is not written), then committed once (cache updated). Blocks of up
    to 128 tokens take the single-kernel path, 200 the chunked one; bf16 I/O at d_inner 256."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_block

    D, N = 256, 16
    A, Dv, bias = I.make_params(D, N)
    rng = np.random.default_rng(G)
    h0 = rng.standard_normal((1, D, N)).astype(np.float32)
    h = f32_dev(h0)
    for r in range(5):
        inp = I.make_activations(1, G, D, N, "bf16", seed=7, xz_seed=500 + r)
        inp.update(A=A, D=Dv, dt_bias=bias)
        dev = upload(inp, "bf16")
        commit = r == 4
        out = bimamba_scan_block(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                                 dev["dt_bias"], h_in=h, h_out=h if commit else None)
        torch.cuda.synchronize()
        want, want_h = oracle.scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                         inp["dt_bias"], h0)
        err = rel_err(to_host64(out), want)
        say(f"block G={G} run {r}{' (commit)' if commit else ''}: out {err:.3e}")
        assert err <= tol_for("bf16")
        if not commit:
            assert np.array_equal(to_host64(h), h0.astype(np.float64)), "a re-run without h_out wrote the cache"
    assert rel_err(to_host64(h), want_h) <= 1e-5


def test_block_in_place_and_null_state():
    """h_out == h_in (in-place commit) and h_in == NULL (zero cache) behave like separate buffers."""
    import torch

    inp = _case(1, 40, 64, 16, "f32")
    dev = upload(inp, "f32")
    h = torch.zeros(1, 64, 16, device="cuda")
    out1 = _block_call(dev, dev, None, h)  # NULL h_in means zeros
    h2 = torch.zeros_like(h)
    out2 = _block_call(dev, dev, h2, h2)  # in place from zeros
    assert torch.equal(out1, out2) and torch.equal(h, h2)
    out3 = _block_call(dev, dev, h2, h2)  # in place from the committed state
    want, want_h = oracle.scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                     inp["dt_bias"], to_host64(h))
    assert rel_err(to_host64(out3), want) <= 1e-4
    assert rel_err(to_host64(h2), want_h) <= 1e-5


def test_block_sweep_workload():
    """batch 1, L 32768, d_inner 4096, d_state 16, bf16, blocks of 32: all 1024 blocks chained through
    the fp32 cache; outputs and the cached state at every block boundary on a channel subset."""
    import torch

    w = I.WORKLOADS["block_32k_bf16"]
    G = w.block_len
    say("block sweep: generating inputs")
    inp = _case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype)
    dev = upload(inp, w.io_dtype)
    chan = np.arange(5, w.d_inner, 64)
    h = torch.zeros(w.batch, w.d_inner, w.d_state, device="cuda")
    outs = torch.empty_like(dev["x"])
    hs = []
    say("block sweep: 1024 GPU calls")
    from bidirectional_mamba_selective_amd import bimamba_scan_block

    for b0 in range(0, w.seqlen, G):
        sl = _slice(dev, b0, b0 + G)
        o = bimamba_scan_block(sl["x"], sl["dt"], dev["A"], sl["B"], sl["C"], dev["D"], sl["z"], dev["dt_bias"],
                               h_in=h, h_out=h)
        outs[:, b0:b0 + G] = o
        hs.append(h[:, chan, :].clone())
    torch.cuda.synchronize()
    got = to_host64(outs)[:, :, chan]
    got_h = np.stack([to_host64(t) for t in hs])
    say("block sweep: oracle on the channel subset")
    sub = {k: (inp[k][:, :, chan] if k in ("x", "dt", "z") else inp[k]) for k in ("x", "dt", "z", "B", "C")}
    hh = None
    want = np.empty_like(got)
    want_h = np.empty_like(got_h)
    for i, b0 in enumerate(range(0, w.seqlen, G)):
        o, hh = oracle.scan_block(sub["x"][:, b0:b0 + G], sub["dt"][:, b0:b0 + G], inp["A"][chan],
                                  sub["B"][:, b0:b0 + G], sub["C"][:, b0:b0 + G], inp["D"][chan],
                                  sub["z"][:, b0:b0 + G], inp["dt_bias"][chan], hh)
        want[:, b0:b0 + G] = o
        want_h[i] = hh
    e_out = rel_err(got, want)
    e_h = max(rel_err(got_h[i], want_h[i]) for i in range(len(hs)))
    say(f"block sweep: out rel err {e_out:.3e}, worst cached-state rel err {e_h:.3e}")
    assert e_out <= tol_for(w.io_dtype)
    assert e_h <= 1e-5


def test_batched_workload_calls():
    """batch 8, L 8192, d_inner 2048, d_state 16, bf16: denoising calls 0, 63 and 127, each with fresh
    seeded x and z (seed 1000 + call) and fixed dt, B, C, A, D, dt_bias; channel-subset oracle."""
    w = I.WORKLOADS["batched_8k_bf16"]
    A, Dv, bias = I.make_params(w.d_inner, w.d_state)
    chan = np.arange(11, w.d_inner, 128)
    for s in (0, 63, 127):
        say(f"batched call {s}: generating inputs")
        inp = I.make_activations(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, seed=1, xz_seed=1000 + s)
        inp.update(A=A, D=Dv, dt_bias=bias)
        dev = upload(inp, w.io_dtype)
        from tests.gpu_util import run_fwd

        out = to_host64(run_fwd(dev))[:, :, chan]
        want = oracle_fwd(inp, chan=chan)
        err = rel_err(out, want)
        say(f"batched call {s}: rel err {err:.3e}")
        assert err <= tol_for(w.io_dtype)


def test_staged_entry_point_matches_fused():
    """Stages 0, 1, 2 in order produce exactly the fused call's output."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_fwd, bimamba_scan_fwd_stage, \
        bimamba_scan_fwd_workspace_bytes

    inp = _case(2, 3000, 256, 16, "bf16")
    dev = upload(inp, "bf16")
    fused = bimamba_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"], dev["dt_bias"])
    ws = torch.empty(bimamba_scan_fwd_workspace_bytes(2, 3000, 256, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["x"])
    for st in range(3):
        bimamba_scan_fwd_stage(st, dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                               dev["dt_bias"], out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)


@pytest.mark.parametrize("shift", [-60.0, 60.0])
@pytest.mark.parametrize("G", [32, 100, 200])
def test_block_delta_limits(shift, G):
    """The block step with dt_bias shifted far down (the cached state passes through unchanged) and
    far up (the state forgets the cache), on the single-kernel and the chunked path (fp32 I/O)."""
    import torch

    inp = _case(2, G, 128, 16, "f32", seed=G + 7)
    inp["dt_bias"] = (inp["dt_bias"] + np.float32(shift)).astype(np.float32)
    h0 = np.random.default_rng(G + 7).standard_normal((2, 128, 16)).astype(np.float32)
    dev = upload(inp, "f32")
    h_in = f32_dev(h0)
    h_out = torch.empty_like(h_in)
    out = to_host64(_block_call(dev, dev, h_in, h_out))
    want, want_h = oracle.scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                     inp["dt_bias"], h0)
    e_out, e_h = rel_err(out, want), rel_err(to_host64(h_out), want_h)
    say(f"block G={G} dt_bias{shift:+.0f}: out {e_out:.3e} h_out {e_h:.3e}")
    assert e_out <= 1e-4 and e_h <= 1e-5
