"""Parity at sizes where every activation tensor exceeds 4 GiB (byte offsets past 32 bits: tile bases,
boundary states, outputs) and, for the convolution, at the largest channel count the library accepts.

The activations are drawn on the device (`inputs.device_normals`: the recipe's distributions, torch's
seeded generator, rounded once to the I/O dtype), since drawing 10^10 values on the host would take
minutes; the oracle gets the sampled channels or heads of those same bits.  Output channel d (head h)
depends only on channel d (head h) and the shared B, C (pins P9, S6, and the convolution's depthwise
form), so the oracle on a sample is exact for it.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import f32_dev, rel_err, say, to_host64, tol_for, torch_mod

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
    err = rel_err(got, want)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= tol_for("bf16")


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
    ef, er = rel_err(gf, wf), rel_err(gr, wr)
    say(f"  rel err fwd {ef:.3e} rev {er:.3e}")
    assert ef <= 1e-5 and er <= 1e-5


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
    err = rel_err(got, want)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= tol_for("bf16")
