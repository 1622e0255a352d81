"""GPU parity of the short causal / anti-causal convolution against the fp64 oracle, through the C ABI.

Also runs the convolution ahead of the untied scan (each direction's filter output is that direction's x),
compared with the oracle's convolution followed by its untied scan.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs
from tests.gpu_util import check, f32_dev, say, to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu


def _case(batch, L, C, io, seed=0):
    rng = np.random.default_rng(seed)
    u = inputs.round_to(rng.standard_normal((batch, L, C)).astype(np.float32), io)
    w_f = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    w_r = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    b_f = (0.1 * rng.standard_normal(C)).astype(np.float32)
    b_r = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return dict(u=u, w_f=w_f, w_r=w_r, b_f=b_f, b_r=b_r)


def _dev(cs, io):
    d = {"u": to_dev(cs["u"], io)}
    d.update({k: f32_dev(cs[k]) for k in ("w_f", "w_r", "b_f", "b_r")})
    return d


@pytest.mark.parametrize("batch,L,C,io", [(1, 1, 4, "f32"), (2, 77, 64, "f32"), (1, 130, 12, "f32"),
                                          (1, 300, 4096, "bf16"), (2, 1000, 256, "bf16"), (3, 64, 1028, "bf16")])
def test_conv_bidir(batch, L, C, io):
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_conv1d_bidir

    torch = torch_mod()
    say(f"conv bidir batch={batch} L={L} C={C} {io}")
    cs = _case(batch, L, C, io)
    d = _dev(cs, io)
    f, r = bimamba_conv1d_bidir(d["u"], d["w_f"], d["b_f"], d["w_r"], d["b_r"])
    torch.cuda.synchronize()
    wf, wr = oracle.conv_bidir(cs["u"], cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"])
    kind = "conv_f32" if io == "f32" else "bf16"
    check(to_host64(f), wf, kind, f"conv {batch}x{L}x{C} {io} fwd")
    check(to_host64(r), wr, kind, f"conv {batch}x{L}x{C} {io} rev")


@pytest.mark.parametrize("mode", ["fwd_only", "rev_only", "no_silu", "tied", "no_bias"])
def test_conv_variants(mode):
    import oracle
    from bidirectional_mamba_selective_amd import FLAG_NO_SILU, bimamba_conv1d_bidir

    torch = torch_mod()
    say(f"conv variant {mode}")
    cs = _case(2, 150, 128, "f32", seed=3)
    d = _dev(cs, "f32")
    act = mode != "no_silu"
    flags = 0 if act else FLAG_NO_SILU
    w_r, b_r, wr_h, br_h = d["w_r"], d["b_r"], cs["w_r"], cs["b_r"]
    if mode == "tied":
        w_r, b_r, wr_h, br_h = d["w_f"], d["b_f"], cs["w_f"], cs["b_f"]
    b_f, bf_h = d["b_f"], cs["b_f"]
    if mode == "no_bias":
        b_f = b_r = bf_h = br_h = None
    f, r = bimamba_conv1d_bidir(d["u"], None if mode == "rev_only" else d["w_f"], b_f,
                                None if mode == "fwd_only" else w_r, b_r, flags=flags)
    torch.cuda.synchronize()
    if mode != "rev_only":
        check(to_host64(f), oracle.conv_causal(cs["u"], cs["w_f"], bf_h, act=act), "conv_f32", f"conv {mode} fwd")
    else:
        assert f is None
    if mode != "fwd_only":
        check(to_host64(r), oracle.conv_anticausal(cs["u"], wr_h, br_h, act=act), "conv_f32", f"conv {mode} rev")
    else:
        assert r is None


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_blocks_chained(io):
    """Blocks of 1, 2, 5, 32, 64 and 100 tokens chained through the cache (in place for some), against the
    oracle's block step; the chained forward outputs also equal the full-sequence causal filter."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_conv1d_block

    torch = torch_mod()
    say(f"conv blocks {io}")
    C = 256
    sizes = [1, 2, 5, 32, 64, 100]
    cs = _case(2, sum(sizes), C, io, seed=5)
    d = _dev(cs, io)
    cache_dev = to_dev(np.zeros((2, 3, C), np.float32), io)
    cache_h = None
    pos = 0
    kind = "conv_f32" if io == "f32" else "bf16"
    for n, G in enumerate(sizes):
        blk = d["u"][:, pos:pos + G].contiguous()
        in_place = n % 2 == 0
        cout = cache_dev if in_place else torch.empty_like(cache_dev)
        f, r = bimamba_conv1d_block(blk, d["w_f"], d["b_f"], d["w_r"], d["b_r"],
                                    cache_in=cache_dev if n > 0 else None, cache_out=cout)
        torch.cuda.synchronize()
        wf, wr, wc = oracle.conv_block(cs["u"][:, pos:pos + G], cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"], cache_h)
        check(to_host64(f), wf, kind, f"conv block {n} fwd")
        check(to_host64(r), wr, kind, f"conv block {n} rev")
        assert np.array_equal(to_host64(cout), wc), f"block {n} cache"  # the cache is a copy of inputs
        cache_dev, cache_h = cout, wc
        pos += G


def test_conv_full_size_sampled():
    """The 1.3B layer's conv shape (4096 channels) at L = 65536, bf16; 24 sampled channels compared in full."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_conv1d_bidir

    torch = torch_mod()
    say("conv L=65536 C=4096 bf16")
    cs = _case(1, 65536, 4096, "bf16", seed=9)
    d = _dev(cs, "bf16")
    f, r = bimamba_conv1d_bidir(d["u"], d["w_f"], d["b_f"], d["w_r"], d["b_r"])
    torch.cuda.synchronize()
    ch = np.random.default_rng(1).choice(4096, 24, replace=False)
    wf, wr = oracle.conv_bidir(cs["u"][:, :, ch], cs["w_f"][ch], cs["b_f"][ch], cs["w_r"][ch], cs["b_r"][ch])
    check(to_host64(f[:, :, torch.from_numpy(ch).cuda()]), wf, "bf16", "conv 64k fwd")
    check(to_host64(r[:, :, torch.from_numpy(ch).cuda()]), wr, "bf16", "conv 64k rev")


def test_conv_then_untied_scan():
    """Each direction's filter output becomes that direction's x of the untied scan (fp32 I/O)."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_conv1d_bidir, bimamba_scan_fwd_untied

    torch = torch_mod()
    say("conv -> untied scan")
    nb, L, D, N = 1, 200, 64, 16
    cs = _case(nb, L, D, "f32", seed=11)
    d = _dev(cs, "f32")
    A, Dv, bias = inputs.make_params(D, N)
    act = inputs.make_activations(nb, L, D, N, "f32", seed=4)
    xf, xr = bimamba_conv1d_bidir(d["u"], d["w_f"], d["b_f"], d["w_r"], d["b_r"])
    common = dict(dt=to_dev(act["dt"], "f32"), B=to_dev(act["B"], "f32"), C=to_dev(act["C"], "f32"),
                  z=to_dev(act["z"], "f32"), A=f32_dev(A), D=f32_dev(Dv), dt_bias=f32_dev(bias))
    of, orr = bimamba_scan_fwd_untied(dict(common, x=xf), dict(common, x=xr))
    torch.cuda.synchronize()
    hf, hr = oracle.conv_bidir(cs["u"], cs["w_f"], cs["b_f"], cs["w_r"], cs["b_r"])
    host = dict(dt=act["dt"], B=act["B"], C=act["C"], z=act["z"], A=A, D=Dv, dt_bias=bias)
    want_f, want_r = oracle.scan_fwd_untied(dict(host, x=hf), dict(host, x=hr))
    check(to_host64(of), want_f, "f32", "conv -> untied scan out_f")
    check(to_host64(orr), want_r, "f32", "conv -> untied scan out_r")
