"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call.

The pointer values below are never dereferenced: every call here fails
validation, which happens on the host before anything reaches HIP.
"""
import ctypes
import os
import re

import pytest

from bidirectional_mamba_selective_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bimamba.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbimamba.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bimamba_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    decl = declared_functions()
    assert decl, "no functions found in the header"
    assert sorted(_lib.EXPORTED) == decl
    for name in decl:
        assert hasattr(lib, name), f"{name} is declared but not exported"


def test_version_and_status_strings():
    assert _lib.bimamba_version() == (0 << 16) | (1 << 8) | 0
    assert _lib.status_string(0) == "ok"
    assert "workspace" in _lib.status_string(3)
    assert _lib.status_string(12345) == "unknown status"


def test_workspace_size_is_monotone_and_zero_when_unsupported():
    f = _lib.bimamba_scan_fwd_workspace_bytes
    sizes = [f(1, L, 4096, 16) for L in (1, 16, 17, 1000, 2048, 65536)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert f(1, 1024, 100, 16) == 0  # d_inner not a multiple of 64
    assert f(1, 1024, 64, 17) == 0  # d_state above 16
    assert f(0, 1024, 64, 16) == 0
    assert all(s % 256 == 0 for s in sizes)


BASE = 1 << 30
SPAN = 1 << 26  # far apart, 256-byte aligned fake device addresses


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * SPAN + off)


def call_fwd(**kw):
    lib = _lib.load()
    a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
             out=fake(8), batch=1, L=64, d=64, n=16, io=_lib.BIMAMBA_BF16, flags=0, ws=fake(9), wsb=0, stream=None)
    a.update(kw)
    return lib.bimamba_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], a["out"],
                                a["batch"], a["L"], a["d"], a["n"], a["io"], a["flags"], a["ws"], a["wsb"],
                                a["stream"])


def call_block(**kw):
    lib = _lib.load()
    a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
             h_in=fake(10), h_out=fake(11), out=fake(8), batch=1, L=32, d=64, n=16, io=_lib.BIMAMBA_BF16, flags=0,
             ws=fake(9), wsb=0, stream=None)
    a.update(kw)
    return lib.bimamba_scan_block(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], a["h_in"],
                                  a["h_out"], a["out"], a["batch"], a["L"], a["d"], a["n"], a["io"], a["flags"],
                                  a["ws"], a["wsb"], a["stream"])


INV, UNS, WS = _lib.BIMAMBA_ERR_INVALID_ARGUMENT, _lib.BIMAMBA_ERR_UNSUPPORTED, _lib.BIMAMBA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), INV),
    (dict(dt=None), INV),
    (dict(A=None), INV),
    (dict(B=None), INV),
    (dict(C=None), INV),
    (dict(out=None), INV),
    (dict(z=None), INV),  # z is required unless the gate is off
    (dict(flags=_lib.FLAG_FWD_ONLY | _lib.FLAG_REV_ONLY), INV),
    (dict(flags=64), INV),
    (dict(batch=0), INV),
    (dict(L=0), INV),
    (dict(L=-5), INV),
    (dict(d=0), INV),
    (dict(n=0), INV),
    (dict(d=100), UNS),
    (dict(n=17), UNS),
    (dict(io=2), UNS),
    (dict(batch=70000), UNS),
    (dict(x=fake(0, 8)), INV),  # misaligned activation
    (dict(A=fake(2, 4)), INV),
    (dict(B=fake(3, 1)), INV),  # not even element-aligned
    (dict(out=fake(0, 64)), INV),  # out overlaps x
    (dict(wsb=0), WS),
    (dict(ws=None, wsb=1 << 40), INV),
    (dict(ws=fake(9, 16), wsb=1 << 40), INV),  # workspace not 256-byte aligned
])
def test_scan_fwd_rejects(kw, want):
    assert call_fwd(**kw) == want


def test_stage_entry_point_validates():
    lib = _lib.load()

    def stage(st, **kw):
        a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
                 out=fake(8), ws=fake(9), wsb=0)
        a.update(kw)
        return lib.bimamba_scan_fwd_stage(st, a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"],
                                          a["out"], 1, 64, 64, 16, _lib.BIMAMBA_BF16, 0, a["ws"], a["wsb"], None)

    for bad in (-2, 3, 100):
        assert stage(bad) == INV
    for st in (-1, 0, 1, 2):
        assert stage(st) == WS
        assert stage(st, x=None) == INV


def test_scan_fwd_checks_run_in_order():
    # z may be NULL with NO_GATE: the call then gets as far as the workspace check
    assert call_fwd(z=None, flags=_lib.FLAG_NO_GATE, wsb=0) == WS
    # D and dt_bias are optional
    assert call_fwd(D=None, dt_bias=None, wsb=0) == WS


@pytest.mark.parametrize("kw,want", [
    (dict(h_in=fake(10, 8)), INV),  # misaligned state
    (dict(h_out=fake(10, 256)), INV),  # partial overlap with h_in
    (dict(h_out=fake(8, 0)), INV),  # h_out overlaps out
    (dict(h_in=fake(8, 0), h_out=None), INV),  # h_in overlaps out
    (dict(h_out=fake(0, 0)), INV),  # h_out over x
    (dict(h_out=fake(3, 0)), INV),  # h_out over B
    (dict(h_out=fake(2, 0)), INV),  # h_out over A
    (dict(x=None), INV),
    (dict(L=0), INV),
    (dict(n=20), UNS),
])
def test_scan_block_rejects(kw, want):
    assert call_block(**kw) == want


def test_block_workspace_only_past_the_single_kernel_limit():
    f = _lib.bimamba_scan_block_workspace_bytes
    # blocks of up to 128 tokens run as one kernel and need no workspace
    assert [f(1, g, 4096, 16) for g in (1, 16, 32, 64, 65, 128)] == [0] * 6
    assert f(1, 129, 4096, 16) > 0 and f(2, 200, 64, 16) > 0
    assert f(1, 100, 100, 16) == 0  # unsupported shape


def test_scan_block_allows_in_place_state():
    # a block past the single-kernel limit: the call then stops at the workspace size check
    assert call_block(L=200, h_out=fake(10), wsb=0) == WS  # h_out == h_in is accepted
    assert call_block(L=200, h_in=None, h_out=None, wsb=0) == WS


def call_untied(**kw):
    lib = _lib.load()
    a = dict(xf=fake(0), dtf=fake(1), Af=fake(2), Bf=fake(3), Cf=fake(4), Df=fake(5), zf=fake(6), bf=fake(7),
             of=fake(8), xr=fake(12), dtr=fake(13), Ar=fake(14), Br=fake(15), Cr=fake(16), Dr=fake(17),
             zr=fake(18), br=fake(19), orr=fake(20), flags=0, ws=fake(9), wsb=0)
    a.update(kw)
    return lib.bimamba_scan_fwd_untied(a["xf"], a["dtf"], a["Af"], a["Bf"], a["Cf"], a["Df"], a["zf"], a["bf"],
                                       a["of"], a["xr"], a["dtr"], a["Ar"], a["Br"], a["Cr"], a["Dr"], a["zr"],
                                       a["br"], a["orr"], 1, 64, 64, 16, _lib.BIMAMBA_BF16, a["flags"], a["ws"],
                                       a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(flags=_lib.FLAG_FWD_ONLY), INV),  # only NO_GATE is meaningful here
    (dict(flags=_lib.FLAG_REV_ONLY), INV),
    (dict(zf=None), INV),  # gate without z
    (dict(zr=None), INV),
    (dict(xr=None), INV),
    (dict(of=fake(12)), INV),  # out_f over the reverse set's x
    (dict(orr=fake(3)), INV),  # out_r over the forward set's B
    (dict(orr=fake(8)), INV),  # the two outputs overlap
    (dict(wsb=0), WS),
])
def test_untied_rejects(kw, want):
    assert call_untied(**kw) == want


def test_untied_checks_run_in_order():
    # without the gate both z may be NULL; the call then stops at the workspace check
    assert call_untied(zf=None, zr=None, flags=_lib.FLAG_NO_GATE) == WS


def call_ssd(stage=None, **kw):
    lib = _lib.load()
    a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
             out=fake(8), batch=1, L=640, h=4, p=32, n=128, io=_lib.BIMAMBA_BF16, flags=0, ws=fake(9), wsb=0)
    a.update(kw)
    args = (a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], a["out"], a["batch"], a["L"],
            a["h"], a["p"], a["n"], a["io"], a["flags"], a["ws"], a["wsb"], None)
    if stage is None:
        return lib.bimamba_ssd_fwd(*args)
    return lib.bimamba_ssd_fwd_stage(stage, *args)


def test_ssd_workspace_size():
    f = _lib.bimamba_ssd_fwd_workspace_bytes
    sizes = [f(1, L, 120, 32, 128) for L in (1, 64, 65, 512, 2048, 65536)]
    assert all(s > 0 and s % 256 == 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert f(1, 64, 4, 64, 128) == 0  # head size other than 32
    assert f(1, 64, 4, 32, 64) == 0  # state size other than 128
    assert f(0, 64, 4, 32, 128) == 0
    # the B/C tiles and the per-chunk states fit in what the plan promises for the 64K-token layer
    assert f(1, 65536, 120, 32, 128) < 512 << 20


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), INV),
    (dict(dt=None), INV),
    (dict(A=None), INV),
    (dict(B=None), INV),
    (dict(C=None), INV),
    (dict(out=None), INV),
    (dict(z=None), INV),
    (dict(flags=_lib.FLAG_FWD_ONLY | _lib.FLAG_REV_ONLY), INV),
    (dict(flags=64), INV),
    (dict(batch=0), INV),
    (dict(L=0), INV),
    (dict(h=0), INV),
    (dict(io=_lib.BIMAMBA_F32), UNS),  # bf16 I/O only
    (dict(io=7), UNS),
    (dict(p=64), UNS),
    (dict(n=16), UNS),
    (dict(batch=70000), UNS),
    (dict(x=fake(0, 8)), INV),  # activations need 16-byte alignment
    (dict(B=fake(3, 2)), INV),
    (dict(dt=fake(1, 1)), INV),
    (dict(A=fake(2, 2)), INV),
    (dict(out=fake(0, 64)), INV),  # out overlaps x
    (dict(out=fake(1, 0)), INV),  # out overlaps dt
    (dict(wsb=0), WS),
    (dict(ws=None, wsb=1 << 40), INV),
    (dict(ws=fake(9, 16), wsb=1 << 40), INV),
])
def test_ssd_rejects(kw, want):
    assert call_ssd(**kw) == want


def test_ssd_checks_run_in_order_and_stages_validate():
    assert call_ssd(z=None, flags=_lib.FLAG_NO_GATE) == WS
    assert call_ssd(D=None, dt_bias=None) == WS
    for bad in (-1, 4, 99):
        assert call_ssd(stage=bad) == INV
    for st in range(4):
        assert call_ssd(stage=st) == WS
        assert call_ssd(stage=st, x=None) == INV


def call_conv(block=False, **kw):
    lib = _lib.load()
    a = dict(u=fake(0), w_f=fake(1), b_f=fake(2), w_r=fake(3), b_r=fake(4), cin=fake(5), cout=fake(6), of=fake(7),
             orr=fake(8), batch=1, L=100, c=64, k=4, io=_lib.BIMAMBA_BF16, flags=0)
    a.update(kw)
    if block:
        return lib.bimamba_conv1d_block(a["u"], a["w_f"], a["b_f"], a["w_r"], a["b_r"], a["cin"], a["cout"], a["of"],
                                        a["orr"], a["batch"], a["L"], a["c"], a["k"], a["io"], a["flags"], None)
    return lib.bimamba_conv1d_bidir(a["u"], a["w_f"], a["b_f"], a["w_r"], a["b_r"], a["of"], a["orr"], a["batch"],
                                    a["L"], a["c"], a["k"], a["io"], a["flags"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(u=None), INV),
    (dict(of=None, orr=None), INV),  # no direction requested
    (dict(w_f=None), INV),  # forward output without its filter
    (dict(w_r=None), INV),
    (dict(batch=0), INV),
    (dict(L=0), INV),
    (dict(c=0), INV),
    (dict(k=0), INV),
    (dict(k=3), UNS),  # only width 4
    (dict(c=62), UNS),  # channels in groups of 4
    (dict(c=(1 << 22) + 4), UNS),  # a tile's rows must fit one buffer resource
    (dict(io=5), UNS),
    (dict(batch=70000), UNS),
    (dict(flags=_lib.FLAG_NO_GATE), INV),
    (dict(u=fake(0, 4)), INV),  # bf16 rows need 8-byte alignment
    (dict(io=_lib.BIMAMBA_F32, of=fake(7, 8)), INV),  # fp32 needs 16
    (dict(w_f=fake(1, 2)), INV),
    (dict(of=fake(0, 64)), INV),  # output over the input
    (dict(orr=fake(7, 0)), INV),  # the two outputs overlap
    (dict(of=fake(3, 0)), INV),  # output over the reverse filter
])
def test_conv_rejects(kw, want):
    assert call_conv(**kw) == want


def test_conv_cache_arguments():
    # block: cache_out over u or an output, or partly over cache_in, is rejected (only rejected calls are made
    # here: an accepted one would launch)
    assert call_conv(block=True, cout=fake(0, 8)) == INV
    assert call_conv(block=True, cout=fake(7, 16)) == INV
    assert call_conv(block=True, cin=fake(6, 8)) == INV  # partial overlap of the two caches
    assert call_conv(block=True, of=fake(5, 0)) == INV  # output over cache_in


def test_binding_counts_workspace_bytes():
    import torch

    assert _lib._bytes_of(None) == 0
    assert _lib._bytes_of(torch.empty(10, dtype=torch.uint8)) == 10
    assert _lib._bytes_of(torch.empty(10, dtype=torch.float32)) == 40  # any dtype: bytes, not elements
    with pytest.raises(ValueError):
        _lib._bytes_of(torch.empty(4, 4, dtype=torch.uint8).t())
    # a host tensor as the workspace of a device call is refused before its address reaches the library
    assert _lib._nbytes(None, torch.device("cuda:0")) == 0
    with pytest.raises(ValueError):
        _lib._nbytes(torch.empty(16, dtype=torch.uint8), torch.device("cuda:0"))


def call_ssd_block(**kw):
    lib = _lib.load()
    a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
             h_in=fake(10), h_out=fake(11), out=fake(8), batch=1, L=100, h=4, p=32, n=128, io=_lib.BIMAMBA_BF16,
             flags=0, ws=fake(9), wsb=0)  # past one run: a valid call stops at the workspace check
    a.update(kw)
    return lib.bimamba_ssd_block(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], a["h_in"],
                                 a["h_out"], a["out"], a["batch"], a["L"], a["h"], a["p"], a["n"], a["io"], a["flags"],
                                 a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), INV),
    (dict(L=0), INV),
    (dict(n=64), UNS),
    (dict(h_in=fake(10, 2)), INV),  # misaligned state
    (dict(h_out=fake(10, 256)), INV),  # partial overlap with h_in
    (dict(h_out=fake(8, 0)), INV),  # h_out over out
    (dict(h_out=fake(0, 0)), INV),  # h_out over x
    (dict(h_out=fake(3, 0)), INV),  # h_out over B
    (dict(h_in=fake(8, 0), h_out=None), INV),  # h_in over out
    (dict(flags=_lib.FLAG_REV_ONLY), INV),  # no forward state to cache
    (dict(wsb=0), WS),
    (dict(h_out=fake(10), wsb=0), WS),  # in-place commit accepted (stops at the workspace check)
    (dict(h_in=None, h_out=None, wsb=0), WS),
    (dict(flags=_lib.FLAG_REV_ONLY, h_out=None, wsb=0), WS),
])
def test_ssd_block_rejects(kw, want):
    assert call_ssd_block(**kw) == want


def test_ssd_block_workspace():
    # blocks of at most one 64-token run take the single-kernel path and need no workspace
    assert [_lib.bimamba_ssd_block_workspace_bytes(2, g, 8, 32, 128) for g in (1, 32, 64)] == [0, 0, 0]
    assert _lib.bimamba_ssd_block_workspace_bytes(2, 100, 8, 32, 128) == \
        _lib.bimamba_ssd_fwd_workspace_bytes(2, 100, 8, 32, 128) > 0


def call_fwd_wide(d, n=16, io=_lib.BIMAMBA_BF16, L=1):
    """scan_fwd with fake tensors 1 GiB apart (room for activations of tens of millions of channels)."""
    lib = _lib.load()

    def p(i):
        return ctypes.c_void_p((1 << 40) + i * (1 << 30))

    return lib.bimamba_scan_fwd(p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), 1, L, d, n, io, 0, p(9), 0, None)


def test_scan_rejects_channels_past_32bit_buffer_offsets():
    """The chunked kernels address a tile's token rows and a boundary's d_state state rows through buffer
    resources of at most 2^31 - 1 bytes with 32-bit offsets: d_inner <= 33554368 at d_state 16."""
    edge, past = 33554368, 33554432
    BF16, F32 = _lib.BIMAMBA_BF16, _lib.BIMAMBA_F32
    assert call_fwd_wide(edge) == WS  # accepted: stops at the workspace size
    assert call_fwd_wide(past) == UNS  # d_state rows of fp32 states exceed 2^31 - 1 bytes
    assert call_fwd_wide(edge, io=F32) == WS
    assert call_fwd_wide(past, io=F32, n=8) == UNS  # 16 token rows of fp32 exceed 2^31 - 1 bytes
    assert call_fwd_wide(past, io=BF16, n=8) == WS  # bf16 rows and 8 state rows still fit
    assert call_fwd_wide(2 * past, io=BF16, n=4) == UNS  # 16 bf16 token rows of 2^26 channels: 2^31 bytes
    f = _lib.bimamba_scan_fwd_workspace_bytes
    assert f(1, 1, edge, 16) > 0 and f(1, 1, past, 16) == 0


def test_scan_block_rejects_cache_overlapping_workspace():
    """Past the single-kernel limit the staging and summary kernels write the workspace before the carry
    kernel reads h_in: a workspace over h_in (or h_out) is rejected."""
    assert call_block(L=200, ws=fake(10), wsb=1 << 40) == INV  # over h_in
    assert call_block(L=200, ws=fake(11), wsb=1 << 40) == INV  # over h_out
    # with h_in NULL the workspace may sit where h_in was (h_out is 64 MiB further on): the call then gets
    # as far as launching, which the fake pointers must not reach, so only the rejections are exercised here


@pytest.mark.parametrize("target", ["x", "dt", "A", "B", "C", "D", "z", "dt_bias"])
def test_workspace_over_an_input_is_rejected(target):
    """The kernels write the workspace while others still read the inputs, so a workspace that overlaps
    any input is rejected before any HIP call (scan, untied directions, a block past the single-kernel
    limit, the Mamba-2 heads)."""
    idx = dict(x=0, dt=1, A=2, B=3, C=4, D=5, z=6, dt_bias=7)[target]
    assert call_fwd(ws=fake(idx), wsb=1 << 40) == INV
    assert call_block(L=200, ws=fake(idx), wsb=1 << 40) == INV
    assert call_ssd(ws=fake(idx), wsb=1 << 40) == INV
    # untied directions: the forward set sits at fake(0..7), the reverse set at fake(12..19)
    assert call_untied(ws=fake(idx), wsb=1 << 40) == INV
    assert call_untied(ws=fake(idx + 12), wsb=1 << 40) == INV


def test_ssd_rejects_head_counts_past_the_output_buffer_range():
    lib = _lib.load()
    f = lib.bimamba_ssd_fwd_workspace_bytes
    assert f(1, 64, 1 << 18, 32, 128) > 0
    assert f(1, 64, (1 << 18) + 1, 32, 128) == 0


def test_noalloc_validates_and_rejects_problems_past_its_scratch():
    """bimamba_scan_fwd_noalloc: the checks of bimamba_scan_fwd, then a problem whose workspace exceeds the
    256 MiB scratch array is rejected before any HIP call."""
    lib = _lib.load()

    def call(**kw):
        a = dict(x=fake(0), dt=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6), dt_bias=fake(7),
                 out=fake(8), batch=1, L=64, d=64, n=16, io=_lib.BIMAMBA_BF16, flags=0)
        a.update(kw)
        return lib.bimamba_scan_fwd_noalloc(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"],
                                            a["out"], a["batch"], a["L"], a["d"], a["n"], a["io"], a["flags"], None)

    assert call(x=None) == INV
    assert call(d=100) == UNS
    assert call(flags=_lib.FLAG_FWD_ONLY | _lib.FLAG_REV_ONLY) == INV
    big = _lib.bimamba_scan_fwd_workspace_bytes(1, 16384, 4096, 16)
    assert big > 256 << 20
    # 16384 tokens of 4096 channels: the activations are 128 MiB apart, so the overlap checks pass
    lib2 = lib

    def p(i):
        return ctypes.c_void_p((1 << 40) + i * (1 << 30))

    st = lib2.bimamba_scan_fwd_noalloc(p(0), p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), 1, 16384, 4096, 16,
                                       _lib.BIMAMBA_BF16, 0, None)
    assert st == _lib.BIMAMBA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in _lib.status_string(st)


def call_ssd_conv(**kw):
    lib = _lib.load()
    # 2 heads of 32 and 128 states: stream rows of 320 channels; tensors 64 MiB apart
    a = dict(xf=fake(0), cwf=fake(1), cbf=fake(2), dtf=fake(3), Af=fake(4), Df=fake(5), zf=fake(6), bf=fake(7),
             of=fake(8), xr=fake(12), cwr=fake(13), cbr=fake(14), dtr=fake(15), Ar=fake(16), Dr=fake(17),
             zr=fake(18), br=fake(19), orr=fake(20), batch=1, L=64, nh=2, hd=32, ns=128, dconv=4,
             io=_lib.BIMAMBA_BF16, flags=0, ws=fake(9), wsb=0)
    a.update(kw)
    return lib.bimamba_ssd_conv_untied(a["xf"], a["cwf"], a["cbf"], a["dtf"], a["Af"], a["Df"], a["zf"], a["bf"],
                                       a["of"], a["xr"], a["cwr"], a["cbr"], a["dtr"], a["Ar"], a["Dr"], a["zr"],
                                       a["br"], a["orr"], a["batch"], a["L"], a["nh"], a["hd"], a["ns"], a["dconv"],
                                       a["io"], a["flags"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(of=None, orr=None), INV),  # neither layer
    (dict(dconv=3), UNS),
    (dict(dconv=0), INV),
    (dict(hd=16), UNS),
    (dict(ns=64), UNS),
    (dict(io=_lib.BIMAMBA_F32), UNS),
    (dict(flags=_lib.FLAG_FWD_ONLY), INV),  # the directions are chosen by the outputs given
    (dict(dtf=None), INV),
    (dict(Ar=None), INV),
    (dict(zf=None), INV),  # gate without z
    (dict(xf=fake(0, 8)), INV),  # misaligned stream
    (dict(of=fake(12)), INV),  # out_f over the reverse layer's stream
    (dict(orr=fake(8)), INV),  # the outputs overlap
    (dict(of=fake(1)), INV),  # out_f over the forward layer's conv taps
    (dict(wsb=0), WS),
])
def test_ssd_conv_untied_rejects(kw, want):
    assert call_ssd_conv(**kw) == want


def test_ssd_conv_untied_checks_run_in_order():
    # one layer alone, no convolution, no gate, no D or bias: the call gets as far as the workspace check
    assert call_ssd_conv(orr=None, xr=None, dtr=None, Ar=None, cwf=None, cbf=None, zf=None, Df=None, bf=None,
                         flags=_lib.FLAG_NO_GATE) == WS
    assert call_ssd_conv(of=None, xf=None, dtf=None, Af=None) == WS


def test_ssd_conv_untied_limits_the_stream_to_32bit_offsets():
    # 2 heads: 320 channels, 640 bytes per token
    lib = _lib.load()

    def p(i):
        return ctypes.c_void_p((1 << 42) + i * (1 << 33))

    def call(L, cw):
        ptr = [p(i) for i in range(18)]
        ptr[1] = cw(1)
        ptr[10] = cw(10)
        return lib.bimamba_ssd_conv_untied(*ptr, 1, L, 2, 32, 128, 4, _lib.BIMAMBA_BF16, 0, p(30), 0, None)

    assert call(3355443, lambda i: p(i)) == UNS  # the stream (+ 256) passes 2^31 - 1 bytes
    assert call(3355442, lambda i: p(i)) == WS  # just below
    assert call(3355443, lambda i: None) == WS  # without the convolution there is no such limit
