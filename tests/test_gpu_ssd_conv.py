"""GPU parity of the Mamba-2 layers with untied directions and their short convolution fused into the scan's
loads (bimamba_ssd_conv_untied), through the C ABI, against the oracle's convolution followed by its scan.

Each direction is its own layer (Section 3.2: two independent layers, the reverse one on the flipped sequence;
Section 4.1 Table 8: untied, width 4; Appendix C Table 12: Conv1d over the xBC stream before the scan).  The
reference is oracle.conv_causal (forward layer) or oracle.conv_anticausal (reverse layer), rounded to bf16 as
the entry point states (the convolution's output takes the I/O precision, as when it is stored between two
passes), split into x, B, C and fed to oracle.ssd_scan_fwd with one direction kept.  Bars: the "ssd" bars of
tests/gpu_util.py (bf16 output, bf16 matrix-core operands: each element within its rounding plus three bf16
roundings of the magnitudes of its terms), and "ssd_pair" where two results of the HIP path are compared.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs
from tests.gpu_util import check, f32_dev, say, ssd_magnitudes, to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu

P, N = 32, 128


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()
    yield


def _upload(inp, conv=True):
    d = {k: to_dev(inp[k], "bf16") for k in ("xbc", "dt", "z")}
    d.update({k: f32_dev(inp[k]) for k in ("A", "D", "dt_bias")})
    if conv:
        d.update(cw=f32_dev(inp["cw"]), cb=f32_dev(inp["cb"]))
    return d


def reference(inp, direction, conv=True, gate=True, use_D=True, use_bias=True, heads=None):
    """The oracle's convolution (of the direction), rounded to bf16, then its one-direction scan; heads
    selects a subset of heads (the stream's B and C channels are shared by all heads).  Returns (out, cols,
    the magnitudes of each output element's terms)."""
    import oracle

    nh = inp["A"].shape[0]
    hp = nh * P
    u = inp["xbc"]
    if conv:
        f = oracle.conv_causal if direction == "f" else oracle.conv_anticausal
        u = f(u, inp["cw"], inp["cb"])
        u = inputs.round_to(u.astype(np.float32), "bf16")
    hs = list(range(nh)) if heads is None else list(heads)
    cols = np.concatenate([np.arange(h * P, (h + 1) * P) for h in hs])
    x, B, C = u[:, :, cols], u[:, :, hp:hp + N], u[:, :, hp + N:hp + 2 * N]
    args = (x, inp["dt"][:, :, hs], inp["A"][hs], B, C, inp["D"][hs] if use_D else None,
            inp["z"][:, :, cols] if gate else None, inp["dt_bias"][hs] if use_bias else None)
    kw = dict(gate=gate, fwd=direction == "f", rev=direction == "r")
    return oracle.ssd_scan_fwd(*args, **kw), cols, ssd_magnitudes(*args, **kw)


def run(fwd, rev, flags=0):
    from bidirectional_mamba_selective_amd import bimamba_ssd_conv_untied

    torch = torch_mod()
    of, orr = bimamba_ssd_conv_untied(fwd, rev, flags=flags)
    torch.cuda.synchronize()
    return of, orr


@pytest.mark.parametrize("batch,L,nh", [(1, 64, 2), (1, 1, 3), (1, 5, 2), (2, 200, 3), (1, 777, 4), (2, 4160, 2)])
def test_layers_with_conv(batch, L, nh):
    say(f"ssd conv layers batch={batch} L={L} heads={nh}")
    f = inputs.make_ssd_layer_inputs(batch, L, nh, seed=L + 1, param_seed=0)
    r = inputs.make_ssd_layer_inputs(batch, L, nh, seed=L + 2, param_seed=3)
    of, orr = run(_upload(f), _upload(r))
    want, _, mag = reference(f, "f")
    check(to_host64(of), want, "ssd", f"conv layers {batch}x{L}x{nh} forward", mag=mag)
    want, _, mag = reference(r, "r")
    check(to_host64(orr), want, "ssd", f"conv layers {batch}x{L}x{nh} reverse", mag=mag)


@pytest.mark.parametrize("mode", ["no_conv", "no_gate", "no_D_no_bias", "forward_only", "reverse_only"])
def test_layer_variants(mode):
    say(f"ssd conv layer variant {mode}")
    f = inputs.make_ssd_layer_inputs(2, 333, 3, seed=7, param_seed=1)
    r = inputs.make_ssd_layer_inputs(2, 333, 3, seed=8, param_seed=2)
    conv = mode != "no_conv"
    gate = mode != "no_gate"
    use = mode != "no_D_no_bias"
    df, dr = _upload(f, conv), _upload(r, conv)
    for d in (df, dr):
        if not gate:
            d["z"] = None
        if not use:
            d["D"] = d["dt_bias"] = None
    of, orr = run(None if mode == "reverse_only" else df, None if mode == "forward_only" else dr,
                  flags=0 if gate else 1)
    if mode != "reverse_only":
        want, _, mag = reference(f, "f", conv, gate, use, use)
        check(to_host64(of), want, "ssd", f"variant {mode} forward", mag=mag)
    else:
        assert of is None
    if mode != "forward_only":
        want, _, mag = reference(r, "r", conv, gate, use, use)
        check(to_host64(orr), want, "ssd", f"variant {mode} reverse", mag=mag)
    else:
        assert orr is None


def test_one_direction_walks_match_the_bidirectional_kernels():
    """Without the convolution, each layer equals bimamba_ssd_fwd with FWD_ONLY / REV_ONLY on the same x, B, C
    (the same mathematics through different kernels and decompositions), to the "ssd_pair" bars."""
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd

    torch = torch_mod()
    f = inputs.make_ssd_layer_inputs(1, 5000, 4, seed=21, param_seed=4)
    d = _upload(f, conv=False)
    of, orr = run(d, d)
    hp = 4 * P
    xs = d["xbc"]
    x, B, C = xs[:, :, :hp].contiguous(), xs[:, :, hp:hp + N].contiguous(), xs[:, :, hp + N:].contiguous()
    wf = bimamba_ssd_fwd(x, d["dt"], d["A"], B, C, d["D"], d["z"], d["dt_bias"], flags=2)
    wr = bimamba_ssd_fwd(x, d["dt"], d["A"], B, C, d["D"], d["z"], d["dt_bias"], flags=4)
    torch.cuda.synchronize()
    check(to_host64(of), to_host64(wf), "ssd_pair", "forward layer vs bidirectional kernels (FWD_ONLY)",
          mag=reference(f, "f", conv=False)[2])
    check(to_host64(orr), to_host64(wr), "ssd_pair", "reverse layer vs bidirectional kernels (REV_ONLY)",
          mag=reference(f, "r", conv=False)[2])


def test_fused_equals_convolution_then_scan_on_the_gpu():
    """The fused call against the two-pass GPU pipeline: bimamba_conv1d_bidir on each layer's stream, then the
    same entry point without the convolution."""
    from bidirectional_mamba_selective_amd import bimamba_conv1d_bidir

    f = inputs.make_ssd_layer_inputs(1, 3000, 4, seed=31, param_seed=5)
    r = inputs.make_ssd_layer_inputs(1, 3000, 4, seed=32, param_seed=6)
    df, dr = _upload(f), _upload(r)
    of, orr = run(df, dr)
    uf, _ = bimamba_conv1d_bidir(df["xbc"], df["cw"], df["cb"], None, None)
    _, ur = bimamba_conv1d_bidir(dr["xbc"], None, None, dr["cw"], dr["cb"])
    pf, pr = run(dict(df, xbc=uf, cw=None, cb=None), dict(dr, xbc=ur, cw=None, cb=None))
    check(to_host64(of), to_host64(pf), "ssd_pair", "fused vs two-pass, forward layer", mag=reference(f, "f")[2])
    check(to_host64(orr), to_host64(pr), "ssd_pair", "fused vs two-pass, reverse layer", mag=reference(r, "r")[2])


def test_full_shape_sampled_heads():
    """The 1.3B layer's shape: 120 heads of 32, state 128, the 4096-channel xBC stream, L = 65536 (chunks of 61
    runs), both layers; heads 0, 60 and 119 of each in full against the oracle."""
    torch = torch_mod()
    nb, L, H = 1, 65536, 120
    xs = H * P + 2 * N
    say("ssd conv layers full shape: drawing inputs on the device")
    sets = []
    for s in (51, 52):
        d = inputs.device_normals({"xbc": (nb, L, xs), "dt": (nb, L, H), "z": (nb, L, H * P)}, seed=s,
                                  io_dtype="bf16", scales={"dt": 0.5})
        A, Dv, bias = inputs.make_ssd_params(H, seed=s - 50)
        cw = inputs.normal(s, "conv_w", (xs, 4), 0.5, "f32")
        cb = inputs.normal(s, "conv_b", (xs,), 0.1, "f32")
        d.update(A=f32_dev(A), D=f32_dev(Dv), dt_bias=f32_dev(bias), cw=f32_dev(cw), cb=f32_dev(cb))
        sets.append((d, dict(A=A, D=Dv, dt_bias=bias, cw=cw, cb=cb)))
    of, orr = run(sets[0][0], sets[1][0])
    for (d, host), out, direction in ((sets[0], of, "f"), (sets[1], orr, "r")):
        for h in (0, 60, 119):
            chan = np.concatenate([np.arange(h * P, (h + 1) * P), np.arange(H * P, xs)])
            ci = torch.from_numpy(chan).cuda()
            inp = dict(xbc=to_host64(d["xbc"][:, :, ci]), dt=to_host64(d["dt"][:, :, h:h + 1]),
                       z=to_host64(d["z"][:, :, h * P:(h + 1) * P]), A=host["A"][h:h + 1], D=host["D"][h:h + 1],
                       dt_bias=host["dt_bias"][h:h + 1], cw=host["cw"][chan], cb=host["cb"][chan])
            want, _, mag = reference(inp, direction)
            cols = torch.from_numpy(np.arange(h * P, (h + 1) * P)).cuda()
            check(to_host64(out[:, :, cols]), want, "ssd", f"full shape {direction} head {h}", mag=mag)
