"""Calls on several streams at once, and workspaces the binding allocates for a caller's stream.

The library keeps no state between calls: each call's kernels read its inputs and write its own output and
workspace, and every kernel computes each output element in a fixed order (no atomics, no cross-workgroup
reductions).  So calls running side by side on different streams give the same bits as the same calls run
one after another.  The second test covers the binding's allocation rule: a workspace and an output that
the caller does not pass are allocated on the stream the kernels run on, so that the caching allocator
cannot hand their memory to other work before those kernels are done.
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


def _scan_set(seed, L=8192, D=2048, N=16):
    d = I.device_normals({"x": (1, L, D), "dt": (1, L, D), "z": (1, L, D), "B": (1, L, N), "C": (1, L, N)},
                         seed=seed, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = I.make_params(D, N, seed=seed, a_jitter=0.2 if seed % 2 else 0.0)
    d.update(A=f32_dev(A), D=f32_dev(Dv), dt_bias=f32_dev(bias))
    return d


def _ssd_set(seed, L=4096, H=24):
    d = I.device_normals({"x": (1, L, H * 32), "dt": (1, L, H), "z": (1, L, H * 32), "B": (1, L, 128),
                          "C": (1, L, 128)}, seed=seed, io_dtype="bf16", scales={"dt": 0.5})
    A, Dv, bias = I.make_ssd_params(H, seed=seed)
    d.update(A=f32_dev(A), D=f32_dev(Dv), dt_bias=f32_dev(bias))
    return d


def _args(d):
    return d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"]


def test_concurrent_streams_match_serial():
    """Two chunked scans (geometric and general A), a Mamba-2 call and a chain of 8 block steps, each on a
    stream of its own and launched together three times over, against the same calls run one after another
    on the default stream: bit-identical outputs and caches."""
    import bidirectional_mamba_selective_amd as bm

    torch = torch_mod()
    dev = torch.device("cuda")
    s1, s2 = _scan_set(31), _scan_set(32)
    q = _ssd_set(33)
    blk = _scan_set(34, L=256, D=4096)
    G = 32
    # the blocks' inputs as contiguous tensors made here, before any side stream runs
    blocks = [{k: blk[k][:, b0:b0 + G].contiguous() for k in ("x", "dt", "z", "B", "C")} for b0 in range(0, 256, G)]

    def run_all(streams, outs):
        """Enqueue every call; streams = None runs them all on the current stream."""
        st = streams or [None] * 4
        bm.bimamba_scan_fwd(*_args(s1), out=outs["s1"], workspace=outs["w1"], stream=st[0])
        bm.bimamba_scan_fwd(*_args(s2), out=outs["s2"], workspace=outs["w2"], stream=st[1])
        bm.bimamba_ssd_fwd(*_args(q), out=outs["q"], workspace=outs["wq"], stream=st[2])
        for i, sl in enumerate(blocks):
            bm.bimamba_scan_block(sl["x"], sl["dt"], blk["A"], sl["B"], sl["C"], blk["D"], sl["z"], blk["dt_bias"],
                                  h_in=outs["h"], h_out=outs["h"], out=outs["b"][i], stream=st[3])

    def new_outs():
        o = {"s1": torch.empty_like(s1["x"]), "s2": torch.empty_like(s2["x"]), "q": torch.empty_like(q["x"]),
             "h": torch.zeros(1, 4096, 16, dtype=torch.float32, device=dev),
             "b": [torch.empty(1, G, 4096, dtype=torch.bfloat16, device=dev) for _ in range(256 // G)],
             "w1": torch.empty(bm.bimamba_scan_fwd_workspace_bytes(1, 8192, 2048, 16), dtype=torch.uint8, device=dev),
             "w2": torch.empty(bm.bimamba_scan_fwd_workspace_bytes(1, 8192, 2048, 16), dtype=torch.uint8, device=dev),
             "wq": torch.empty(bm.bimamba_ssd_fwd_workspace_bytes(1, 4096, 24, 32, 128), dtype=torch.uint8,
                               device=dev)}
        return o

    say("streams: serial reference on the default stream")
    ref = new_outs()
    run_all(None, ref)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev) for _ in range(4)]  # default priority
    for rep in range(3):
        say(f"streams: concurrent run {rep}")
        got = new_outs()
        for s_ in streams:
            s_.wait_stream(torch.cuda.current_stream(dev))
        run_all(streams, got)
        torch.cuda.synchronize()
        for k in ("s1", "s2", "q", "h"):
            assert torch.equal(got[k], ref[k]), f"run {rep}: {k} differs from the serial run"
        for i, (a_, b_) in enumerate(zip(got["b"], ref["b"])):
            assert torch.equal(a_, b_), f"run {rep}: block {i} differs from the serial run"


def test_binding_allocates_on_the_callers_stream():
    """Calls on a side stream that let the binding allocate out and the workspace, while the default stream
    keeps allocating and filling tensors of the same sizes (which would take over any block freed too early):
    every output equals the one computed with caller-owned buffers."""
    import bidirectional_mamba_selective_amd as bm

    torch = torch_mod()
    dev = torch.device("cuda")
    s1 = _scan_set(35)
    q = _ssd_set(36)
    ref = bm.bimamba_scan_fwd(*_args(s1))
    ref_q = bm.bimamba_ssd_fwd(*_args(q))
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    nws = bm.bimamba_scan_fwd_workspace_bytes(1, 8192, 2048, 16)
    outs = []
    for rep in range(6):
        o = bm.bimamba_scan_fwd(*_args(s1), stream=side)
        oq = bm.bimamba_ssd_fwd(*_args(q), stream=side)
        outs.append((o, oq))
        # the default stream now allocates and overwrites blocks of the sizes the side stream's calls freed
        junk = [torch.full((nws,), 255, dtype=torch.uint8, device=dev), torch.full_like(s1["x"], 7.0)]
        del junk
    torch.cuda.synchronize()
    for rep, (o, oq) in enumerate(outs):
        assert torch.equal(o, ref), f"call {rep}: scan output differs"
        assert torch.equal(oq, ref_q), f"call {rep}: Mamba-2 output differs"
    say("streams: 6 side-stream calls with binding-allocated buffers equal the reference")
