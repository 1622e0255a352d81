"""Parity at sizes where every activation tensor exceeds 4 GiB (byte offsets past 32 bits: tile bases,
boundary states, outputs), and at the largest sizes the library accepts: the convolution's channel count,
the scan's d_inner (chunked call and block step) and the Mamba-2 head count.

The activations are drawn on the device (`inputs.device_normals`: the recipe's distributions, torch's
seeded generator, rounded once to the I/O dtype), since drawing 10^10 values on the host would take
minutes; the oracle gets the sampled channels or heads of those same bits.  Output channel d (head h)
depends only on channel d (head h) and the shared B, C (pins P9, S6, and the convolution's depthwise
form), so the oracle on a sample is exact for it.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import check, f32_dev, say, ssd_magnitudes, to_host64, torch_mod

pytestmark = pytest.mark.gpu


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_scan_tensors_over_4gib():
    """batch 8, L 65536, d_inner 4096, N 16, bf16: x, dt, z and out are 4 GiB each, the boundary
    states 8 GiB; 12 channels of every batch element and token against the oracle."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_scan_fwd

    torch = torch_mod()
    nb, L, D, N = 8, 65536, 4096, 16
    say(f"scan {nb}x{L}x{D}x{N} bf16: drawing inputs on the device")
    act = I.device_normals({"x": (nb, L, D), "dt": (nb, L, D), "z": (nb, L, D), "B": (nb, L, N), "C": (nb, L, N)},
                           seed=21, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = I.make_params(D, N)
    say("scan over 4 GiB: running")
    out = bimamba_scan_fwd(act["x"], act["dt"], f32_dev(A), act["B"], act["C"], f32_dev(Dv), act["z"], f32_dev(bias))
    torch.cuda.synchronize()
    chan = np.array([0, 5, 63, 64, 1000, 2047, 2048, 3000, 4030, 4093, 4094, 4095])
    ci = torch.from_numpy(chan).cuda()
    got = to_host64(out[:, :, ci])
    hx, hdt, hz = (_host(act[k][:, :, ci]) for k in ("x", "dt", "z"))
    hB, hC = _host(act["B"]), _host(act["C"])
    del out, act
    torch.cuda.empty_cache()
    say("scan over 4 GiB: oracle on 12 channels")
    want = oracle.scan_fwd(hx, hdt, A[chan], hB, hC, Dv[chan], hz, bias[chan])
    check(got, want, "bf16", "scan over 4 GiB")


def test_conv_max_channels_over_4gib():
    """The largest channel count accepted (2^22) in fp32 at L = 300: u and both outputs are 5 GB each;
    the buffer resources of a tile span 67 rows of 16 MiB.  24 channels against the oracle."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_conv1d_bidir

    torch = torch_mod()
    C, L = 1 << 22, 300
    say(f"conv L={L} C={C} f32: drawing inputs on the device")
    d = I.device_normals({"u": (1, L, C), "w_f": (C, 4), "w_r": (C, 4), "b_f": (C,), "b_r": (C,)}, seed=22,
                         io_dtype="f32", scales={"w_f": 0.5, "w_r": 0.5, "b_f": 0.1, "b_r": 0.1})
    f, r = bimamba_conv1d_bidir(d["u"], d["w_f"], d["b_f"], d["w_r"], d["b_r"])
    torch.cuda.synchronize()
    ch = np.array([0, 1, 2, 3, 4, 1023, 1024, 65535, 65536, 1 << 20, (1 << 21) + 7, (1 << 22) - 8, (1 << 22) - 5,
                   (1 << 22) - 4, (1 << 22) - 3, (1 << 22) - 2, (1 << 22) - 1, 12345, 2222222, 3333333, 4000000,
                   4100000, 4194300, 777777])
    ci = torch.from_numpy(ch).cuda()
    gf, gr = to_host64(f[:, :, ci]), to_host64(r[:, :, ci])
    hu = _host(d["u"][:, :, ci])
    hw = {k: _host(d[k][ci]) for k in ("w_f", "w_r", "b_f", "b_r")}
    del f, r, d
    torch.cuda.empty_cache()
    wf, wr = oracle.conv_bidir(hu, hw["w_f"], hw["b_f"], hw["w_r"], hw["b_r"])
    check(gf, wf, "conv_f32", "conv 2^22 channels fwd")
    check(gr, wr, "conv_f32", "conv 2^22 channels rev")


def test_ssd_tensors_over_4gib():
    """Mamba-2 heads at batch 9, L 65536, 120 heads of 32, N 128, bf16: x, z and out are 4.2 GiB each;
    heads 0 and 119 of the first and the last batch element against the oracle."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd

    torch = torch_mod()
    nb, L, H, Pd, N = 9, 65536, 120, 32, 128
    say(f"ssd {nb}x{L} heads {H}x{Pd} N {N} bf16: drawing inputs on the device")
    act = I.device_normals({"x": (nb, L, H * Pd), "dt": (nb, L, H), "z": (nb, L, H * Pd), "B": (nb, L, N),
                            "C": (nb, L, N)}, seed=23, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = I.make_ssd_params(H)
    out = bimamba_ssd_fwd(act["x"], act["dt"], f32_dev(A), act["B"], act["C"], f32_dev(Dv), act["z"], f32_dev(bias))
    torch.cuda.synchronize()
    heads = np.array([0, 119])
    cols = np.concatenate([np.arange(h * Pd, (h + 1) * Pd) for h in heads])
    bsel = torch.tensor([0, nb - 1]).cuda()  # the first and the last batch element (the highest addresses)
    ci, hi = torch.from_numpy(cols).cuda(), torch.from_numpy(heads).cuda()
    got = to_host64(out[bsel][:, :, ci])
    hx, hz = _host(act["x"][bsel][:, :, ci]), _host(act["z"][bsel][:, :, ci])
    hdt = _host(act["dt"][bsel][:, :, hi])
    hB, hC = _host(act["B"][bsel]), _host(act["C"][bsel])
    del out, act
    torch.cuda.empty_cache()
    say("ssd over 4 GiB: oracle on 2 heads")
    want = oracle.ssd_scan_fwd(hx, hdt, A[heads], hB, hC, Dv[heads], hz, bias[heads])
    mag = ssd_magnitudes(hx, hdt, A[heads], hB, hC, Dv[heads], hz, bias[heads])
    check(got, want, "ssd", "ssd over 4 GiB", mag=mag)


# The largest d_inner the scan accepts for an I/O dtype and state size: a tile of 16 token rows, and the
# d_state rows of fp32 states at a tile boundary, each just under 2^31 bytes (the range of one buffer
# resource).  fp32 with 16 states: 16 * d * 4 <= 2^31 - 1 and 16 * d * 4 + 256 <= 2^31 - 1; bf16 with 8
# states: 16 * d * 2 and 8 * d * 4 (+ 256).  d_inner is the largest multiple of 64 under both.
_MAX_CASES = [("f32", 16, 33554368), ("bf16", 8, 67108800)]


@pytest.mark.parametrize("io, N, D", _MAX_CASES, ids=[f"{c[0]}-N{c[1]}" for c in _MAX_CASES])
def test_scan_max_channels(io, N, D):
    """At the largest accepted d_inner, L = 20 (one chunk: a full tile and a ragged one): the chunked call,
    then the block step over the same 20 tokens from a random cache, on 14 channels including the last
    wavefront's, against the oracle (out, and the new cache)."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_scan_block, bimamba_scan_fwd

    torch = torch_mod()
    es = 4 if io == "f32" else 2
    assert 16 * D * es <= 2**31 - 1 and N * D * 4 + 256 <= 2**31 - 1 and D % 64 == 0
    assert 16 * (D + 64) * es > 2**31 - 1 or N * (D + 64) * 4 + 256 > 2**31 - 1  # the next size is refused
    L = 20
    say(f"scan at the largest d_inner: {io} N {N} D {D} L {L}: drawing inputs on the device")
    act = I.device_normals({"x": (1, L, D), "dt": (1, L, D), "z": (1, L, D), "B": (1, L, N), "C": (1, L, N),
                            "h": (1, D, N)}, seed=24, io_dtype=io, scales={"dt": 0.5})
    h_in = act.pop("h").float()
    A, Dv, bias = I.make_params(D, N)
    Ad, Dd, bd = f32_dev(A), f32_dev(Dv), f32_dev(bias)
    chan = np.array([0, 1, 63, 64, 65, 1 << 20, D // 2, D // 2 + 1, 12345678, D - 65, D - 64, D - 63, D - 2, D - 1])
    ci = torch.from_numpy(chan).cuda()
    hx, hdt, hz = (_host(act[k][:, :, ci]) for k in ("x", "dt", "z"))
    hB, hC = _host(act["B"]), _host(act["C"])
    hh = h_in[:, ci, :].double().cpu().numpy()

    say(f"scan at the largest d_inner ({io}): chunked call")
    out = bimamba_scan_fwd(act["x"], act["dt"], Ad, act["B"], act["C"], Dd, act["z"], bd)
    torch.cuda.synchronize()
    got = to_host64(out[:, :, ci])
    del out
    torch.cuda.empty_cache()
    bar = "f32" if io == "f32" else "bf16"
    check(got, oracle.scan_fwd(hx, hdt, A[chan], hB, hC, Dv[chan], hz, bias[chan]), bar,
          f"scan at d_inner {D} ({io}, N {N})")

    say(f"scan at the largest d_inner ({io}): block step")
    h_out = torch.empty_like(h_in)
    out = bimamba_scan_block(act["x"], act["dt"], Ad, act["B"], act["C"], Dd, act["z"], bd, h_in=h_in, h_out=h_out)
    torch.cuda.synchronize()
    got = to_host64(out[:, :, ci])
    got_h = h_out[:, ci, :].double().cpu().numpy()
    del out, h_out, h_in, act
    torch.cuda.empty_cache()
    want, want_h = oracle.scan_block(hx, hdt, A[chan], hB, hC, Dv[chan], hz, bias[chan], h_in=hh)
    check(got, want, bar, f"block step at d_inner {D} ({io}, N {N})")
    check(got_h, want_h, "state", f"block cache at d_inner {D} ({io}, N {N})")


def test_ssd_max_heads():
    """Mamba-2 at the largest head count accepted (2^18 heads of 32 channels), L = 70 (a run and a ragged
    one): a run's output rows span 1 GiB of one buffer resource, the chunk states 8 GiB; 9 heads including
    the last ones against the oracle."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd

    torch = torch_mod()
    H, Pd, N, L = 1 << 18, 32, 128, 70
    say(f"ssd at the largest head count: {H} heads, L {L}: drawing inputs on the device")
    act = I.device_normals({"x": (1, L, H * Pd), "dt": (1, L, H), "z": (1, L, H * Pd), "B": (1, L, N),
                            "C": (1, L, N)}, seed=25, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = I.make_ssd_params(H)
    out = bimamba_ssd_fwd(act["x"], act["dt"], f32_dev(A), act["B"], act["C"], f32_dev(Dv), act["z"], f32_dev(bias))
    torch.cuda.synchronize()
    heads = np.array([0, 1, 7, 8, H // 2 - 1, H // 2, H - 8, H - 2, H - 1])
    cols = np.concatenate([np.arange(h * Pd, (h + 1) * Pd) for h in heads])
    ci, hi = torch.from_numpy(cols).cuda(), torch.from_numpy(heads).cuda()
    got = to_host64(out[:, :, ci])
    hx, hz = _host(act["x"][:, :, ci]), _host(act["z"][:, :, ci])
    hdt = _host(act["dt"][:, :, hi])
    hB, hC = _host(act["B"]), _host(act["C"])
    del out, act
    torch.cuda.empty_cache()
    say("ssd at the largest head count: oracle on 9 heads")
    want = oracle.ssd_scan_fwd(hx, hdt, A[heads], hB, hC, Dv[heads], hz, bias[heads])
    mag = ssd_magnitudes(hx, hdt, A[heads], hB, hC, Dv[heads], hz, bias[heads])
    check(got, want, "ssd", f"ssd at {H} heads", mag=mag)
