"""Every entry point captured into a HIP graph and replayed.

The library allocates nothing, issues no memset and keeps no host-side state between calls, so a call
captured once replays correctly on whatever the captured buffers hold at replay time.  Each case captures
one call (or a chain of calls) on a side stream, then three times: new inputs (and a new cache) are copied
into the captured buffers by eager work on the replay stream, the graph is replayed, the host synchronises,
and the graph's outputs are compared with the eager call on the same inputs, bit for bit.
"""
import pytest

from bidirectional_mamba_selective_amd import inputs as I
from tests.gpu_util import f32_dev, say, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bidirectional_mamba_selective_amd import load

    load()
    yield


def _capture(fn):
    """fn(stream) captured once into a graph (after one eager warm-up call on the capture stream)."""
    torch = torch_mod()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        fn(gs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            fn(gs)
    torch.cuda.synchronize()
    return g


def _replays(name, g, buffers, draw, graph_outs, eager):
    """Three rounds: copy draw(rep) into `buffers`, replay, compare graph_outs() with eager() (bit for bit)."""
    torch = torch_mod()
    for rep in range(3):
        new = draw(rep)
        for k, t in new.items():
            buffers[k].copy_(t)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in graph_outs()]
        want = eager()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"{name}: replay {rep}, output {i} differs from the eager call"
    say(f"graphs: {name}: 3 replays equal the eager calls")


def _act(shapes, seed, io="bf16", scales=None):
    return I.device_normals(shapes, seed=seed, io_dtype=io, scales=scales or {"dt": 0.5})


def test_graph_scan_and_untied():
    import bidirectional_mamba_selective_amd as bm

    torch = torch_mod()
    L, D, N = 4096, 1024, 16
    shp = {"x": (1, L, D), "dt": (1, L, D), "z": (1, L, D), "B": (1, L, N), "C": (1, L, N)}
    buf = _act(shp, 40)
    A, Dv, bias = (f32_dev(a) for a in I.make_params(D, N, a_jitter=0.2))
    out = torch.empty_like(buf["x"])
    ws = torch.empty(bm.bimamba_scan_fwd_workspace_bytes(1, L, D, N), dtype=torch.uint8, device="cuda")
    args = lambda d: (d["x"], d["dt"], A, d["B"], d["C"], Dv, d["z"], bias)  # noqa: E731
    g = _capture(lambda s: bm.bimamba_scan_fwd(*args(buf), out=out, workspace=ws, stream=s))
    _replays("scan", g, buf, lambda r: _act(shp, 41 + r), lambda: [out],
             lambda: [bm.bimamba_scan_fwd(*args(buf))])

    rev = _act(shp, 50)
    A2, D2, b2 = (f32_dev(a) for a in I.make_params(D, N, seed=3))
    fset = dict(buf, A=A, D=Dv, dt_bias=bias)
    rset = dict(rev, A=A2, D=D2, dt_bias=b2)
    of, orr = torch.empty_like(out), torch.empty_like(out)
    g2 = _capture(lambda s: bm.bimamba_scan_fwd_untied(fset, rset, out_f=of, out_r=orr, workspace=ws, stream=s))
    both = {**{"f" + k: v for k, v in buf.items()}, **{"r" + k: v for k, v in rev.items()}}

    def draw2(r):
        a, b = _act(shp, 51 + r), _act(shp, 61 + r)
        return {**{"f" + k: v for k, v in a.items()}, **{"r" + k: v for k, v in b.items()}}

    _replays("untied scan", g2, both, draw2, lambda: [of, orr], lambda: list(bm.bimamba_scan_fwd_untied(fset, rset)))


def test_graph_block_chains():
    """Four 32-token block steps chained through the cache in place, and one 200-token block (chunked path,
    with its workspace), captured together; the cache is redrawn before each replay."""
    import bidirectional_mamba_selective_amd as bm

    torch = torch_mod()
    D, N, G = 4096, 16, 32
    shp = {"x": (1, 4 * G + 200, D), "dt": (1, 4 * G + 200, D), "z": (1, 4 * G + 200, D),
           "B": (1, 4 * G + 200, N), "C": (1, 4 * G + 200, N)}
    full = _act(shp, 70)
    A, Dv, bias = (f32_dev(a) for a in I.make_params(D, N))
    keys = ("x", "dt", "z", "B", "C")
    spans = [(i * G, G) for i in range(4)] + [(4 * G, 200)]
    blk = [{k: full[k][:, s:s + n].contiguous() for k in keys} for s, n in spans]
    h = torch.zeros(1, D, N, dtype=torch.float32, device="cuda")
    h_big = torch.zeros_like(h)
    outs = [torch.empty_like(b["x"]) for b in blk]
    ws = torch.empty(bm.bimamba_scan_block_workspace_bytes(1, 200, D, N), dtype=torch.uint8, device="cuda")

    def chain(s, hh, hb, oo):
        for i, b in enumerate(blk[:4]):
            bm.bimamba_scan_block(b["x"], b["dt"], A, b["B"], b["C"], Dv, b["z"], bias, h_in=hh, h_out=hh, out=oo[i],
                                  stream=s)
        b = blk[4]
        bm.bimamba_scan_block(b["x"], b["dt"], A, b["B"], b["C"], Dv, b["z"], bias, h_in=hb, h_out=hb, out=oo[4],
                              workspace=ws, stream=s)

    g = _capture(lambda s: chain(s, h, h_big, outs))
    bufs = {f"{k}{i}": blk[i][k] for i in range(5) for k in keys}
    bufs.update(h=h, h_big=h_big)

    def draw(r):
        d = {}
        for i, (s, n) in enumerate(spans):
            a = _act({k: (1, n, D if k in ("x", "dt", "z") else N) for k in keys}, 71 + 10 * r + i)
            d.update({f"{k}{i}": a[k] for k in keys})
        hh = _act({"h": (1, D, N), "hb": (1, D, N)}, 99 + r, io="f32")
        d.update(h=hh["h"], h_big=hh["hb"])
        return d

    def eager():
        # the eager chain starts from the cache the replay started from (redrawn, then advanced by the replay)
        hh, hb = start["h"].clone(), start["h_big"].clone()
        oo = [torch.empty_like(o) for o in outs]
        chain(torch.cuda.current_stream(), hh, hb, oo)
        return oo + [hh, hb]

    start = {}

    def draw_and_keep(r):
        d = draw(r)
        start.update(h=d["h"].clone(), h_big=d["h_big"].clone())
        return d

    _replays("block chains", g, bufs, draw_and_keep, lambda: outs + [h, h_big], eager)


def test_graph_ssd_and_conv():
    """The Mamba-2 call, its block step from a cache, the convolution, its block step, and the fused untied
    Mamba-2 layers with their convolution."""
    import bidirectional_mamba_selective_amd as bm

    torch = torch_mod()
    L, H, P, N = 2048, 16, 32, 128
    shp = {"x": (1, L, H * P), "dt": (1, L, H), "z": (1, L, H * P), "B": (1, L, N), "C": (1, L, N)}
    buf = _act(shp, 80)
    A, Dv, bias = (f32_dev(a) for a in I.make_ssd_params(H))
    out = torch.empty_like(buf["x"])
    ws = torch.empty(bm.bimamba_ssd_fwd_workspace_bytes(1, L, H, P, N), dtype=torch.uint8, device="cuda")
    args = lambda d: (d["x"], d["dt"], A, d["B"], d["C"], Dv, d["z"], bias)  # noqa: E731
    g = _capture(lambda s: bm.bimamba_ssd_fwd(*args(buf), out=out, workspace=ws, stream=s))
    _replays("ssd", g, buf, lambda r: _act(shp, 81 + r), lambda: [out], lambda: [bm.bimamba_ssd_fwd(*args(buf))])

    G = 32
    bshp = {k: (1, G) + v[2:] for k, v in shp.items()}
    bb = _act(bshp, 90)
    hin = torch.zeros(1, H, P, N, dtype=torch.float32, device="cuda")
    hout = torch.empty_like(hin)
    bout = torch.empty_like(bb["x"])
    wsb = torch.empty(max(bm.bimamba_ssd_block_workspace_bytes(1, G, H, P, N), 1), dtype=torch.uint8, device="cuda")
    g2 = _capture(lambda s: bm.bimamba_ssd_block(*args(bb), h_in=hin, h_out=hout, out=bout, workspace=wsb, stream=s))
    bbuf = dict(bb, h=hin)

    def draw2(r):
        d = _act(bshp, 91 + r)
        d["h"] = _act({"h": (1, H, P, N)}, 95 + r, io="f32")["h"]
        return d

    def eager2():
        ho = torch.empty_like(hout)
        o = bm.bimamba_ssd_block(*args(bb), h_in=hin, h_out=ho)
        return [o, ho]

    _replays("ssd block", g2, bbuf, draw2, lambda: [bout, hout], eager2)

    C = 4096
    u = _act({"u": (1, L, C)}, 100)
    wf, wr = f32_dev(I.normal(1, "conv_w", (C, 4), 0.5)), f32_dev(I.normal(2, "conv_w", (C, 4), 0.5))
    bf_, br_ = f32_dev(I.normal(1, "conv_b", (C,), 0.1)), f32_dev(I.normal(2, "conv_b", (C,), 0.1))
    of, orr = torch.empty_like(u["u"]), torch.empty_like(u["u"])
    g3 = _capture(lambda s: bm.bimamba_conv1d_bidir(u["u"], wf, bf_, wr, br_, out_f=of, out_r=orr, stream=s))
    _replays("conv", g3, u, lambda r: _act({"u": (1, L, C)}, 101 + r), lambda: [of, orr],
             lambda: list(bm.bimamba_conv1d_bidir(u["u"], wf, bf_, wr, br_)))

    ub = _act({"u": (1, G, C), "c": (1, 3, C)}, 110)
    cache_out = torch.empty_like(ub["c"])
    obf, obr = torch.empty_like(ub["u"]), torch.empty_like(ub["u"])
    g4 = _capture(lambda s: bm.bimamba_conv1d_block(ub["u"], wf, bf_, wr, br_, cache_in=ub["c"], cache_out=cache_out,
                                                    out_f=obf, out_r=obr, stream=s))

    def eager4():
        co = torch.empty_like(cache_out)
        f, r = bm.bimamba_conv1d_block(ub["u"], wf, bf_, wr, br_, cache_in=ub["c"], cache_out=co)
        return [f, r, co]

    _replays("conv block", g4, ub, lambda r: _act({"u": (1, G, C), "c": (1, 3, C)}, 111 + r),
             lambda: [obf, obr, cache_out], eager4)

    xs = H * P + 2 * N
    sets = []
    for s_ in (120, 121):
        d = _act({"xbc": (1, L, xs), "dt": (1, L, H), "z": (1, L, H * P)}, s_)
        A_, D_, b_ = (f32_dev(a) for a in I.make_ssd_params(H, seed=s_))
        d.update(A=A_, D=D_, dt_bias=b_, cw=f32_dev(I.normal(s_, "conv_w", (xs, 4), 0.5)),
                 cb=f32_dev(I.normal(s_, "conv_b", (xs,), 0.1)))
        sets.append(d)
    f, r = sets
    lf, lr = torch.empty(1, L, H * P, dtype=torch.bfloat16, device="cuda"), torch.empty(
        1, L, H * P, dtype=torch.bfloat16, device="cuda")
    g5 = _capture(lambda s: bm.bimamba_ssd_conv_untied(f, r, out_f=lf, out_r=lr, workspace=ws, stream=s))
    both = {"fx": f["xbc"], "fz": f["z"], "rx": r["xbc"], "rz": r["z"]}

    def draw5(rep):
        a = _act({"fx": (1, L, xs), "fz": (1, L, H * P), "rx": (1, L, xs), "rz": (1, L, H * P)}, 130 + rep)
        return a

    _replays("ssd conv layers", g5, both, draw5, lambda: [lf, lr], lambda: list(bm.bimamba_ssd_conv_untied(f, r)))
