"""GPU parity of the Mamba-2 (SSD) scan: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output; the long cases run all 120 heads on the GPU
and compare sampled heads in full against the oracle run on those heads alone
(heads are independent, a fact the oracle's head-independence pin fixes), and
one run at L = 65536 compares every output, the oracle run in shards of heads
by host processes.
"""
import numpy as np
import pytest

from bidirectional_mamba_selective_amd import inputs
from tests.gpu_util import check, f32_dev, say, ssd_magnitudes, to_dev, to_host64, torch_mod

pytestmark = pytest.mark.gpu

# Bars (tests/gpu_util.py BARS): "ssd" for the bf16 output (normwise 2e-2, every element within the rounding of
# its bf16 value plus three bf16 roundings of the sum of the magnitudes of its terms, which the matrix-core
# products' bf16 operands cost); "ssd_state" for the fp32 cache, whose increments are matrix-core products too.  A block of up to 64
# tokens runs as one kernel whose products take each fp32 operand as a pair of bf16 values (the rounded value
# and its residual), so its output is held to the "bf16" bars (its own rounding) and its cache to the
# "ssd_split_state" bars.


def _block_bars(G):
    return ("bf16", "ssd_split_state") if G <= 64 else ("ssd", "ssd_state")


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


def _mag(inp, heads=None, gate=True, fwd=True, rev=True, use_D=True, use_bias=True):
    """The magnitudes of each output element's terms (ssd_magnitudes) on the heads _oracle compares."""
    nh = inp["A"].shape[0]
    hs = list(range(nh)) if heads is None else list(heads)
    cols = np.concatenate([np.arange(h * 32, (h + 1) * 32) for h in hs])
    return ssd_magnitudes(inp["x"][:, :, cols], inp["dt"][:, :, hs], inp["A"][hs], inp["B"], inp["C"],
                          inp["D"][hs] if use_D else None, inp["z"][:, :, cols] if gate else None,
                          inp["dt_bias"][hs] if use_bias else None, gate=gate, fwd=fwd, rev=rev)


@pytest.mark.parametrize("batch,L,nh", [(1, 64, 2), (1, 1, 3), (2, 200, 3), (1, 513, 4), (1, 1100, 2), (2, 4160, 2)])
def test_ssd_small_full_compare(batch, L, nh):
    say(f"ssd parity batch={batch} L={L} heads={nh}")
    inp = _inputs(batch, L, nh)
    got = _run(_upload(inp))
    want, _ = _oracle(inp)
    check(got, want, "ssd", f"ssd batch={batch} L={L} heads={nh}", mag=_mag(inp))


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
    check(got, want, "ssd", f"ssd flags={flags}", mag=_mag(inp, **kw))


def test_ssd_optional_params():
    say("ssd D=None, dt_bias=None")
    inp = _inputs(1, 300, 2, seed=6)
    got = _run(_upload(inp), use_D=False, use_bias=False)
    want, _ = _oracle(inp, use_D=False, use_bias=False)
    check(got, want, "ssd", "ssd D=None dt_bias=None", mag=_mag(inp, use_D=False, use_bias=False))


def test_ssd_delta_to_zero_limit():
    """dt_bias = -30: Delta ~ 1e-13, the output is 2 D x silu(z) to bf16 rounding."""
    say("ssd delta -> 0")
    inp = _inputs(1, 256, 2, seed=7)
    inp["dt_bias"] = np.full(2, -30.0, dtype=np.float32)
    got = _run(_upload(inp))
    x, z = inp["x"].astype(np.float64), inp["z"].astype(np.float64)
    want = 2.0 * x * z / (1.0 + np.exp(-z))
    check(got, want, "bf16", "ssd delta -> 0")


@pytest.mark.parametrize("L", [13312, 65536])
def test_ssd_all_heads_sampled(L):
    """120 heads at the 1.3B layer's shape (chunks of 13 and 61 runs).  Sampled heads are compared in full."""
    say(f"ssd 120 heads L={L}")
    inp = _inputs(1, L, 120, seed=2)
    got = _run(_upload(inp))
    assert np.all(np.isfinite(got))
    for heads in (([0], [57], [119]) if L < 50000 else ([0], [119])):
        want, cols = _oracle(inp, heads=heads)
        check(got[:, :, cols], want, "ssd", f"ssd L={L} head {heads[0]}", mag=_mag(inp, heads=heads))


def test_ssd_full_width():
    """All 120 heads at L = 65536 over the whole output (251 million values) against the oracle run on the
    host in shards of heads, by worker processes (heads are independent given the shared B, C)."""
    from tests.gpu_util import oracle_sharded

    L, H, Pd = 65536, 120, 32
    say(f"ssd full width: {H} heads L={L}")
    inp = _inputs(1, L, H, seed=2)
    got = _run(_upload(inp))

    def heads_last(d, hs):
        # the oracle's output and the magnitudes of its terms, heads on the last axis
        pair = np.stack([_oracle(d, heads=hs)[0], _mag(d, heads=hs)])
        return pair.reshape(2, 1, L, len(hs), Pd).transpose(0, 1, 2, 4, 3)

    say("ssd full width: oracle on 120 heads in host processes")
    pair = oracle_sharded(heads_last, inp, H, (2, 1, L, Pd, H)).transpose(0, 1, 2, 4, 3).reshape(2, 1, L, H * Pd)
    check(got, pair[0], "ssd", f"ssd (all {L} x {H * Pd} outputs)", mag=pair[1])


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
    Bars by path (_block_bars): one kernel up to 64 tokens, the chunked kernels beyond."""
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
    m_out, m_h = ssd_magnitudes(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                inp["z"] if gate else None, inp["dt_bias"], h0, gate=gate, fwd=True,
                                rev=not (flags & 2))
    out_bar, cache_bar = _block_bars(G)
    check(to_host64(out), want, out_bar, f"ssd block G={G} flags={flags} out", mag=m_out)
    check(to_host64(h_out), want_h, cache_bar, f"ssd block G={G} flags={flags} cache", mag=m_h)


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
    mag_f = ssd_magnitudes(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, None, inp["dt_bias"],
                           gate=False, fwd=True, rev=False)
    mh_host = np.zeros((nb, nh, 32, 128))
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
        m_out, m_h = ssd_magnitudes(hb["x"], hb["dt"], inp["A"], hb["B"], hb["C"], inp["D"], hb["z"],
                                    inp["dt_bias"], mh_host)
        out_bar, cache_bar = _block_bars(G)
        check(to_host64(out), want, out_bar, f"ssd block chain G={G} block {k} out", mag=m_out)
        check(to_host64(h), want_h, cache_bar, f"ssd block chain G={G} block {k} cache", mag=m_h)
        check(to_host64(out_f), full_f[:, sl], out_bar, f"ssd block chain G={G} block {k} forward vs full scan",
              mag=mag_f[:, sl])
        h_host, mh_host = want_h, m_h


def test_ssd_full_shape_ssm_only():
    """All 120 heads at L = 65536 (chunks of 61 runs) with D = NULL and no gate, so only the state-space part
    is compared: the carries across 17 chunks and the reverse sweep's partial output cannot hide behind the
    skip term.  Heads 0, 60 and 119 in full against the oracle on those heads."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_fwd

    torch = torch_mod()
    nb, L, H, Pd, N = 1, 65536, 120, 32, 128
    say("ssd full shape ssm-only: drawing inputs on the device")
    act = inputs.device_normals({"x": (nb, L, H * Pd), "dt": (nb, L, H), "B": (nb, L, N), "C": (nb, L, N)},
                                seed=41, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = inputs.make_ssd_params(H)
    out = bimamba_ssd_fwd(act["x"], act["dt"], f32_dev(A), act["B"], act["C"], None, None, f32_dev(bias), flags=1)
    torch.cuda.synchronize()
    for h in (0, 60, 119):
        cols = np.arange(h * Pd, (h + 1) * Pd)
        ci = torch.from_numpy(cols).cuda()
        got = to_host64(out[:, :, ci])
        hx, hdt = to_host64(act["x"][:, :, ci]), to_host64(act["dt"][:, :, h:h + 1])
        want = oracle.ssd_scan_fwd(hx, hdt, A[h:h + 1], to_host64(act["B"]), to_host64(act["C"]), None, None,
                                   bias[h:h + 1], gate=False)
        mag = ssd_magnitudes(hx, hdt, A[h:h + 1], to_host64(act["B"]), to_host64(act["C"]), None, None,
                             bias[h:h + 1], gate=False)
        check(got, want, "ssd", f"ssd full shape ssm-only head {h}", mag=mag)


def test_ssd_block_long_chain():
    """Block decoding over 256 blocks of 64 tokens (16384 tokens) with the cache committed in place after
    each block: the cache at every 16th boundary and every block's output against the oracle chained over the
    same blocks, so a cache error that grew from block to block would fail.  8 heads (heads are independent).
    64-token blocks run as one kernel: "ssd_split_state" bars for the cache, "bf16" for the output."""
    import oracle
    from bidirectional_mamba_selective_amd import bimamba_ssd_block

    torch = torch_mod()
    nb, nh, G, nblk = 1, 8, 64, 256
    L = G * nblk
    say(f"ssd block long chain: {nblk} blocks of {G}")
    inp = _inputs(nb, L, nh, seed=88)
    dev = _upload(inp)
    h = torch.zeros(nb, nh, 32, 128, device="cuda")
    outs = torch.empty_like(dev["x"])
    caches = {}
    for k in range(nblk):
        sl = slice(k * G, (k + 1) * G)
        bl = {key: dev[key][:, sl].contiguous() for key in ("x", "dt", "z", "B", "C")}
        outs[:, sl] = bimamba_ssd_block(bl["x"], bl["dt"], dev["A"], bl["B"], bl["C"], dev["D"], bl["z"],
                                        dev["dt_bias"], h_in=h, h_out=h)
        if k % 16 == 15:
            caches[k] = h.clone()
    torch.cuda.synchronize()
    got = to_host64(outs)
    want = np.empty_like(got)
    h_host = None
    worst_cache = 0.0
    for k in range(nblk):
        sl = slice(k * G, (k + 1) * G)
        hb = {key: inp[key][:, sl] for key in ("x", "dt", "z", "B", "C")}
        want[:, sl], h_host = oracle.ssd_scan_block(hb["x"], hb["dt"], inp["A"], hb["B"], hb["C"], inp["D"],
                                                    hb["z"], inp["dt_bias"], h_host)
        if k % 16 == 15:
            r = check(to_host64(caches[k]), h_host, "ssd_split_state", f"ssd long chain cache after block {k}")
            worst_cache = max(worst_cache, r["norm"])
    # every token row of every block (the per-row bar), and the sampled blocks against their own scale
    check(got, want, "bf16", "ssd long chain, all blocks")
    for k in (0, 127, 255):
        check(got[:, k * G:(k + 1) * G], want[:, k * G:(k + 1) * G], "bf16", f"ssd long chain block {k}")
    say(f"ssd long chain: worst cache normwise error over {nblk} blocks {worst_cache:.3e}")
