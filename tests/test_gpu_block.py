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
from tests.gpu_util import check, f32_dev, oracle_fwd, say, to_dev, to_host64, upload

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


def _check_quiet(got, want):
    """The state bars of tests.gpu_util.check without its log line (the sweep checks 1024 caches)."""
    from tests.gpu_util import BARS

    b = BARS["state"]
    d = got - want
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert np.linalg.norm(d) <= b.norm * np.linalg.norm(want)
    assert np.all(np.abs(d) <= b.rel * np.abs(want) + b.abs * rms)


def _slice(dev, b0, b1):
    return {k: dev[k][:, b0:b1].contiguous() for k in ("x", "dt", "z", "B", "C")}


@pytest.mark.parametrize("G", [1, 5, 16, 17, 31, 32, 48, 63, 64, 100, 128, 129, 200])
@pytest.mark.parametrize("flags", [0, NO_GATE, FWD_ONLY, REV_ONLY | NO_GATE])
def test_block_small(G, flags):
    """One block with a random cached state; out and h_out against oracle.scan_block (fp32 I/O).  The sizes
    cover each single-kernel form and its padding: one group (up to 16 tokens), parts of 16 tokens (17-31 and
    32 in two parts, 48, 63 and 64 in four, with a whole part of padding at 48), halves (100, 128), and
    the chunked path past 128."""
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
    check(out, want, "f32", f"block G={G} flags={flags} out")
    check(to_host64(h_out), want_h, "state", f"block G={G} flags={flags} h_out")


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
    check(out, want, "f32", f"block N={N} G={G} jitter={jitter} out")
    check(to_host64(h), want_h, "state", f"block N={N} G={G} jitter={jitter} h_out")


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
        check(to_host64(out), want, "bf16", f"block G={G} run {r}{' (commit)' if commit else ''}")
        if not commit:
            assert np.array_equal(to_host64(h), h0.astype(np.float64)), "a re-run without h_out wrote the cache"
    check(to_host64(h), want_h, "state", f"block G={G} committed cache")


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
    check(to_host64(out3), want, "f32", "block in place out")
    check(to_host64(h2), want_h, "state", "block in place h_out")


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
    check(got, want, w.io_dtype, "block sweep out")
    # every block's output against its own scale, and the cached state at every block boundary
    worst = max(check(got[:, b0:b0 + G], want[:, b0:b0 + G], w.io_dtype, f"block at {b0}")["elem"]
                for b0 in range(0, w.seqlen, 64 * G))
    say(f"block sweep: worst element of the sampled blocks at {worst:.3f} of its bound")
    for i in range(len(hs)):
        if i % 128 == 0 or i == len(hs) - 1:
            check(got_h[i], want_h[i], "state", f"cache after block {i}")
        else:
            _check_quiet(got_h[i], want_h[i])


def _oracle_sweep(inp, chan, G):
    """The oracle's block sweep on channels chan: blocks of G tokens chained through the forward cache.
    Returns [batch, L + N, len(chan)]: the outputs, then the final cache with its state axis first."""
    hh = None
    L = inp["x"].shape[1]
    out = np.empty(inp["x"].shape[:2] + (len(chan),))
    for b0 in range(0, L, G):
        sl = {k: inp[k][:, b0:b0 + G] for k in ("x", "dt", "z", "B", "C")}
        o, hh = oracle.scan_block(sl["x"][:, :, chan], sl["dt"][:, :, chan], inp["A"][chan], sl["B"], sl["C"],
                                  inp["D"][chan], sl["z"][:, :, chan], inp["dt_bias"][chan], hh)
        out[:, b0:b0 + G] = o
    return np.concatenate([out, hh.transpose(0, 2, 1)], axis=1)


def test_block_sweep_full_width():
    """The block workload's 1024-block sweep (L 32768, d_inner 4096, blocks of 32, the cache committed in place)
    over its whole output, every token of every channel, against the oracle's sweep run on the host in
    channel shards; and the final cache over every channel and state."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_block
    from tests.gpu_util import oracle_sharded

    w = I.WORKLOADS["block_32k_bf16"]
    G = w.block_len
    inp = _case(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype)
    dev = upload(inp, w.io_dtype)
    h = torch.zeros(w.batch, w.d_inner, w.d_state, device="cuda")
    outs = torch.empty_like(dev["x"])
    say("block sweep full width: 1024 GPU calls")
    for b0 in range(0, w.seqlen, G):
        sl = _slice(dev, b0, b0 + G)
        outs[:, b0:b0 + G] = bimamba_scan_block(sl["x"], sl["dt"], dev["A"], sl["B"], sl["C"], dev["D"], sl["z"],
                                                dev["dt_bias"], h_in=h, h_out=h)
    torch.cuda.synchronize()
    got = to_host64(outs)
    got_h = to_host64(h)
    say(f"block sweep full width: oracle on {w.d_inner} channels in host processes")
    both = oracle_sharded(lambda d, c: _oracle_sweep(d, c, G), inp, w.d_inner,
                          (w.batch, w.seqlen + w.d_state, w.d_inner))
    check(got, both[:, :w.seqlen], w.io_dtype, f"block sweep (all {w.seqlen} x {w.d_inner} outputs)")
    check(got_h, both[:, w.seqlen:].transpose(0, 2, 1), "state", "block sweep final cache (all channels and states)")


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
        check(out, want, w.io_dtype, f"batched call {s}")


def test_batched_call_full_width():
    """Denoising call 0 of the batched workload (batch 8, L 8192, d_inner 2048, bf16; x, z seeded 1000) over
    its whole output, 134 million elements, against the oracle run on the host in channel shards (exact: a
    channel's output depends only on that channel and the shared B, C) by up to 8 worker processes."""
    from tests.gpu_util import oracle_sharded, run_fwd

    w = I.WORKLOADS["batched_8k_bf16"]
    A, Dv, bias = I.make_params(w.d_inner, w.d_state)
    inp = I.make_activations(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, seed=1, xz_seed=1000)
    inp.update(A=A, D=Dv, dt_bias=bias)
    say("batched call 0, full width: running on the GPU")
    got = to_host64(run_fwd(upload(inp, w.io_dtype)))
    say(f"batched call 0, full width: oracle on {w.d_inner} channels in host processes")
    want = oracle_sharded(lambda d, c: oracle_fwd(d, chan=c), inp, w.d_inner, got.shape)
    check(got, want, w.io_dtype, "batched call 0 (all 8 x 8192 x 2048 outputs)")


def test_batched_workload_all_calls_channel_subset():
    """All 128 denoising calls of the batched workload (batch 8, L 8192, d_inner 2048, bf16), each with fresh
    x and z drawn on the device (torch's generator seeded 1000 + call; dt, B, C drawn once), one workspace
    reused by every call; each call's output on 8 channels of every batch element against the oracle on the
    same bits (a channel's output depends only on that channel and the shared B, C).  The subset moves with
    the call, so the 128 calls cover 1024 different channels."""
    import torch

    from bidirectional_mamba_selective_amd import bimamba_scan_fwd, bimamba_scan_fwd_workspace_bytes

    w = I.WORKLOADS["batched_8k_bf16"]
    A, Dv, bias = I.make_params(w.d_inner, w.d_state)
    fixed = I.device_normals({"dt": (w.batch, w.seqlen, w.d_inner), "B": (w.batch, w.seqlen, w.d_state),
                              "C": (w.batch, w.seqlen, w.d_state)}, seed=1, io_dtype="bf16", scales={"dt": 0.5})
    Ad, Dd, bd = f32_dev(A), f32_dev(Dv), f32_dev(bias)
    ws = torch.empty(bimamba_scan_fwd_workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(w.batch, w.seqlen, w.d_inner, dtype=torch.bfloat16, device="cuda")
    host_fixed = {k: to_host64(fixed[k]) for k in ("B", "C")}
    worst = 0.0
    for s in range(128):
        xz = I.device_normals({"x": (w.batch, w.seqlen, w.d_inner), "z": (w.batch, w.seqlen, w.d_inner)},
                              seed=1000 + s, io_dtype="bf16")
        bimamba_scan_fwd(xz["x"], fixed["dt"], Ad, fixed["B"], fixed["C"], Dd, xz["z"], bd, out=out, workspace=ws)
        chan = (np.arange(8) * 256 + 8 * s + 3) % w.d_inner
        ci = torch.from_numpy(chan).cuda()
        got = to_host64(out[:, :, ci])
        inp = {"x": to_host64(xz["x"][:, :, ci]), "z": to_host64(xz["z"][:, :, ci]),
               "dt": to_host64(fixed["dt"][:, :, ci]), "B": host_fixed["B"], "C": host_fixed["C"], "A": A[chan],
               "D": Dv[chan], "dt_bias": bias[chan]}
        r = check(got, oracle_fwd(inp), "bf16", f"batched call {s}", quiet=s % 32 != 0)
        worst = max(worst, r["elem"])
    say(f"batched workload: all 128 calls, worst element at {worst:.3f} of its bound")


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
    check(out, want, "f32", f"block G={G} dt_bias{shift:+.0f} out")
    check(to_host64(h_out), want_h, "state", f"block G={G} dt_bias{shift:+.0f} h_out")
