"""GPU parity of the Mamba-2 (SSD) scan: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output; the long cases run all 120 heads on the GPU
and compare sampled heads in full against the oracle run on those heads alone
(heads are independent, a fact the oracle's head-independence pin fixes).
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs
from tests.gpu_util import f32_dev, rel_err, say, to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu

TOL = 2e-2  # normwise relative error bar with bf16 I/O
# The block cache is carried in fp32, but its increment sum_j w_j x_j (outer) B_j is a matrix-core product of
# bf16 operands: each weighted x is rounded to bf16 (relative error <= 2^-9 = 1.95e-3 per term), and a sum of
# terms of both signs can amplify that normwise; measured 1.6e-3 - 1.8e-3 when the whole cache is increments.
# The cache is held to 1e-2, half the output's bar.
CACHE_TOL = 1e-2


def _inputs(batch, L, nh, seed=1):
    A, D, dt_bias = inputs.make_ssd_params(nh)
    act = inputs.make_ssd_activations(batch, L, nh, 32, 128, "bf16", seed=seed)
    act.update(A=A, D=D, dt_bias=dt_bias)
    return act


def _upload(inp):
    dev = {k: to_dev(inp[k], "bf16") for k in ("x", "dt", "z", "B", "C")}
    dev.update({k: f32_dev(inp[k]) for k in ("A", "D", "dt_bias")})
    return dev


def _run(dev, flags=0, use_D=True, use_bias=True, use_z=True):
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd

    torch = torch_mod()
    out = bimamba_ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"] if use_D else None,
                          dev["z"] if use_z else None, dev["dt_bias"] if use_bias else None, flags=flags)
    torch.cuda.synchronize()
    return to_host64(out)


def _oracle(inp, heads=None, gate=True, fwd=True, rev=True, use_D=True, use_bias=True):
    import oracle

    nh = inp["A"].shape[0]
    hs = list(range(nh)) if heads is None else list(heads)
    cols = np.concatenate([np.arange(h * 32, (h + 1) * 32) for h in hs])
    return oracle.ssd_scan_fwd(inp["x"][:, :, cols], inp["dt"][:, :, hs], inp["A"][hs], inp["B"], inp["C"],
                               inp["D"][hs] if use_D else None, inp["z"][:, :, cols] if gate else None,
                               inp["dt_bias"][hs] if use_bias else None, gate=gate, fwd=fwd, rev=rev), cols


@pytest.mark.parametrize("batch,L,nh", [(1, 64, 2), (1, 1, 3), (2, 200, 3), (1, 513, 4), (1, 1100, 2), (2, 4160, 2)])
def test_ssd_small_full_compare(batch, L, nh):
    say(f"ssd parity batch={batch} L={L} heads={nh}")
    inp = _inputs(batch, L, nh)
    got = _run(_upload(inp))
    want, _ = _oracle(inp)
    err = rel_err(got, want)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL


@pytest.mark.parametrize("flags,kw", [
    (2, dict(fwd=True, rev=False)),
    (4, dict(fwd=False, rev=True)),
    (1, dict(gate=False)),
    (3, dict(gate=False, fwd=True, rev=False)),
])
def test_ssd_flags(flags, kw):
    say(f"ssd flags={flags}")
    inp = _inputs(1, 777, 3, seed=5)
    got = _run(_upload(inp), flags=flags, use_z=kw.get("gate", True))
    want, _ = _oracle(inp, **kw)
    err = rel_err(got, want)
    say(f"  rel err {err:.3e}")
    assert err <= TOL


def test_ssd_optional_params():
    say("ssd D=None, dt_bias=None")
    inp = _inputs(1, 300, 2, seed=6)
    got = _run(_upload(inp), use_D=False, use_bias=False)
    want, _ = _oracle(inp, use_D=False, use_bias=False)
    assert rel_err(got, want) <= TOL


def test_ssd_delta_to_zero_limit():
    """dt_bias = -30: Delta ~ 1e-13, the output is 2 D x silu(z) to bf16 rounding."""
    say("ssd delta -> 0")
    inp = _inputs(1, 256, 2, seed=7)
    inp["dt_bias"] = np.full(2, -30.0, dtype=np.float32)
    got = _run(_upload(inp))
    x, z = inp["x"].astype(np.float64), inp["z"].astype(np.float64)
    want = 2.0 * x * z / (1.0 + np.exp(-z))
    assert rel_err(got, want) <= 1e-2


@pytest.mark.parametrize("L", [13312, 65536])
def test_ssd_all_heads_sampled(L):
    """120 heads at the 1.3B layer's shape (chunks of 13 and 61 runs).  Sampled heads are compared in full."""
    say(f"ssd 120 heads L={L}")
    inp = _inputs(1, L, 120, seed=2)
    got = _run(_upload(inp))
    assert np.all(np.isfinite(got))
    for heads in (([0], [57], [119]) if L < 50000 else ([0], [119])):
        want, cols = _oracle(inp, heads=heads)
        err = rel_err(got[:, :, cols], want)
        say(f"  head {heads[0]}: rel err {err:.3e}")
        assert err <= TOL


def test_ssd_deterministic_and_staged():
    """Two calls give identical bits, and the four stages run one by one give the same bits again."""
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd, bimamba_ssd_fwd_stage, bimamba_ssd_fwd_workspace_bytes

    torch = torch_mod()
    say("ssd determinism and stages")
    inp = _inputs(1, 5000, 8, seed=3)
    dev = _upload(inp)
    args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"], dev["dt_bias"])
    o1 = bimamba_ssd_fwd(*args)
    o2 = bimamba_ssd_fwd(*args)
    ws = torch.empty(bimamba_ssd_fwd_workspace_bytes(1, 5000, 8, 32, 128), dtype=torch.uint8, device="cuda")
    o3 = torch.empty_like(o1)
    for st in range(4):
        bimamba_ssd_fwd_stage(st, *args, out=o3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o1, o3)


@pytest.mark.parametrize("G", [1, 32, 64, 100, 300])
@pytest.mark.parametrize("flags", [0, 1, 2])
def test_ssd_block_step(G, flags):
    """One block with a random cached state (block-cache decoding, Section 4.3): out and the new cache
    against oracle.ssd_scan_block; flags 0 (both directions, gated), 1 (no gate), 2 (forward only).
    The output is held to the bf16 bar; the cache (carried in fp32, its increments formed by bf16-operand
    products on the matrix cores) to CACHE_TOL."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_block

    torch = torch_mod()
    nb, nh = 2, 3
    say(f"ssd block G={G} flags={flags}")
    inp = _inputs(nb, G, nh, seed=G + 40)
    h0 = np.random.default_rng(G).standard_normal((nb, nh, 32, 128)).astype(np.float32)
    dev = _upload(inp)
    h_in = f32_dev(h0)
    h_out = torch.empty_like(h_in)
    gate = not (flags & 1)
    out = bimamba_ssd_block(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"] if gate else None,
                            dev["dt_bias"], h_in=h_in, h_out=h_out, flags=flags)
    torch.cuda.synchronize()
    want, want_h = oracle.ssd_scan_block(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                         inp["z"] if gate else None, inp["dt_bias"], h0, gate=gate,
                                         fwd=True, rev=not (flags & 2))
    e_out, e_h = rel_err(to_host64(out), want), rel_err(to_host64(h_out), want_h)
    say(f"  out {e_out:.3e} cache {e_h:.3e}")
    assert e_out <= TOL and e_h <= CACHE_TOL


@pytest.mark.parametrize("G", [64, 96])
def test_ssd_block_chain_and_reruns(G):
    """Block decoding over 6 blocks with the cache committed in place (64-token blocks take the
    single-kernel path, 96 the chunked one); before each commit the block is re-run twice without h_out
    (the cache must not change).  Every block's output and the cache at every boundary against the
    oracle; the chained forward-only outputs also equal the full forward scan."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_block

    torch = torch_mod()
    nb, nh, nblk = 1, 4, 6
    L = G * nblk
    inp = _inputs(nb, L, nh, seed=77)
    dev = _upload(inp)
    h = torch.zeros(nb, nh, 32, 128, device="cuda")
    h_host = None
    full_f = oracle.ssd_scan_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, None, inp["dt_bias"],
                                 gate=False, fwd=True, rev=False)
    for k in range(nblk):
        sl = slice(k * G, (k + 1) * G)
        bl = {key: dev[key][:, sl].contiguous() for key in ("x", "dt", "z", "B", "C")}
        hb = {key: inp[key][:, sl] for key in ("x", "dt", "z", "B", "C")}
        before = h.clone()
        for _ in range(2):  # re-runs from the same cache
            bimamba_ssd_block(bl["x"], bl["dt"], dev["A"], bl["B"], bl["C"], dev["D"], bl["z"], dev["dt_bias"],
                              h_in=h, h_out=None)
        torch.cuda.synchronize()
        assert torch.equal(h, before), f"block {k}: a re-run without h_out wrote the cache"
        out = bimamba_ssd_block(bl["x"], bl["dt"], dev["A"], bl["B"], bl["C"], dev["D"], bl["z"], dev["dt_bias"],
                                h_in=h, h_out=h)  # commit in place
        out_f = bimamba_ssd_block(bl["x"], bl["dt"], dev["A"], bl["B"], bl["C"], None, None, dev["dt_bias"],
                                  h_in=before, h_out=None, flags=1 | 2)  # forward only, no gate, no D
        torch.cuda.synchronize()
        want, want_h = oracle.ssd_scan_block(hb["x"], hb["dt"], inp["A"], hb["B"], hb["C"], inp["D"], hb["z"],
                                             inp["dt_bias"], h_host)
        e_out = rel_err(to_host64(out), want)
        e_h = rel_err(to_host64(h), want_h)
        e_f = rel_err(to_host64(out_f), full_f[:, sl])
        say(f"ssd block chain G={G} {k}: out {e_out:.3e} cache {e_h:.3e} forward vs full scan {e_f:.3e}")
        assert e_out <= TOL and e_h <= CACHE_TOL and e_f <= TOL
        h_host = want_h
