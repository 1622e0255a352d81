"""ctypes binding of libbimamba.so.

Argument marshalling only: torch tensors are checked (device, dtype,
contiguity, shape), their data pointers and the current HIP stream are passed
to the C entry points of include/bimamba.h, and a non-zero status raises.
Every step of the scan runs in the library's HIP kernels; there is no other
path.  If the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbimamba.so")

BIMAMBA_OK = 0
BIMAMBA_ERR_INVALID_ARGUMENT = 1
BIMAMBA_ERR_UNSUPPORTED = 2
BIMAMBA_ERR_WORKSPACE_TOO_SMALL = 3
BIMAMBA_ERR_HIP = 4
BIMAMBA_ERR_SCRATCH_TOO_SMALL = 5

BIMAMBA_F32 = 0
BIMAMBA_BF16 = 1

FLAG_NO_GATE = 1
FLAG_FWD_ONLY = 2
FLAG_REV_ONLY = 4
FLAG_NO_SILU = 16

# every symbol include/bimamba.h declares
EXPORTED = (
    "bimamba_version",
    "bimamba_status_string",
    "bimamba_scan_fwd_workspace_bytes",
    "bimamba_scan_fwd",
    "bimamba_scan_fwd_stage",
    "bimamba_scan_fwd_noalloc",
    "bimamba_scan_fwd_untied",
    "bimamba_scan_block_workspace_bytes",
    "bimamba_scan_block",
    "bimamba_ssd_fwd_workspace_bytes",
    "bimamba_ssd_fwd",
    "bimamba_ssd_fwd_stage",
    "bimamba_ssd_block_workspace_bytes",
    "bimamba_ssd_block",
    "bimamba_ssd_conv_untied",
    "bimamba_conv1d_bidir",
    "bimamba_conv1d_block",
)

_lib = None


class BimambaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Load libbimamba.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bidirectional_mamba_selective_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.bimamba_version.restype = ctypes.c_int
    lib.bimamba_version.argtypes = []
    lib.bimamba_status_string.restype = ctypes.c_char_p
    lib.bimamba_status_string.argtypes = [ctypes.c_int]
    lib.bimamba_scan_fwd_workspace_bytes.restype = sz
    lib.bimamba_scan_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.bimamba_scan_block_workspace_bytes.restype = sz
    lib.bimamba_scan_block_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.bimamba_scan_fwd.restype = ctypes.c_int
    lib.bimamba_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_scan_fwd_stage.restype = ctypes.c_int
    lib.bimamba_scan_fwd_stage.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                           ctypes.c_int, ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_scan_fwd_noalloc.restype = ctypes.c_int
    lib.bimamba_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_uint32, vp]
    lib.bimamba_scan_fwd_untied.restype = ctypes.c_int
    lib.bimamba_scan_fwd_untied.argtypes = [vp] * 18 + [i64, i64, i64, i64, ctypes.c_int, ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_scan_block.restype = ctypes.c_int
    lib.bimamba_scan_block.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                       ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_ssd_fwd_workspace_bytes.restype = sz
    lib.bimamba_ssd_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.bimamba_ssd_fwd.restype = ctypes.c_int
    lib.bimamba_ssd_fwd.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_int, ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_ssd_fwd_stage.restype = ctypes.c_int
    lib.bimamba_ssd_fwd_stage.argtypes = [ctypes.c_int] + [vp] * 9 + [i64] * 5 + [ctypes.c_int, ctypes.c_uint32, vp,
                                                                                    sz, vp]
    lib.bimamba_ssd_block_workspace_bytes.restype = sz
    lib.bimamba_ssd_block_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.bimamba_ssd_block.restype = ctypes.c_int
    lib.bimamba_ssd_block.argtypes = [vp] * 11 + [i64] * 5 + [ctypes.c_int, ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_ssd_conv_untied.restype = ctypes.c_int
    lib.bimamba_ssd_conv_untied.argtypes = [vp] * 18 + [i64] * 6 + [ctypes.c_int, ctypes.c_uint32, vp, sz, vp]
    lib.bimamba_conv1d_bidir.restype = ctypes.c_int
    lib.bimamba_conv1d_bidir.argtypes = [vp] * 7 + [i64] * 4 + [ctypes.c_int, ctypes.c_uint32, vp]
    lib.bimamba_conv1d_block.restype = ctypes.c_int
    lib.bimamba_conv1d_block.argtypes = [vp] * 9 + [i64] * 4 + [ctypes.c_int, ctypes.c_uint32, vp]
    _lib = lib
    return lib


def bimamba_version() -> int:
    return load().bimamba_version()


def status_string(status: int) -> str:
    return load().bimamba_status_string(int(status)).decode()


bimamba_status_string = status_string


def bimamba_scan_fwd_workspace_bytes(batch: int, seqlen: int, d_inner: int, d_state: int) -> int:
    return int(load().bimamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state))


def bimamba_scan_block_workspace_bytes(batch: int, block_len: int, d_inner: int, d_state: int) -> int:
    return int(load().bimamba_scan_block_workspace_bytes(batch, block_len, d_inner, d_state))


def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bytes_of(t):
    """Bytes of a caller-provided workspace tensor (any dtype; it must be contiguous); 0 for None."""
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return t.numel() * t.element_size()


def _nbytes(t, device):
    """_bytes_of a workspace that must sit on the call's device (a host tensor's address would reach the kernels)."""
    if t is not None and (not t.is_cuda or t.device != device):
        raise ValueError(f"workspace must be on {device}")
    return _bytes_of(t)


def _io_dtype(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        return BIMAMBA_BF16
    if x.dtype == torch.float32:
        return BIMAMBA_F32
    raise TypeError(f"unsupported I/O dtype {x.dtype}; use torch.bfloat16 or torch.float32")


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _common(x, dt, A, B, C, D, z, dt_bias, out):
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, d_inner]")
    nb, L, nd = x.shape
    ns = A.shape[1] if A.dim() == 2 else -1
    io = x.dtype
    dev = x.device
    _check(x, "x", (nb, L, nd), io, dev)
    _check(dt, "dt", (nb, L, nd), io, dev)
    _check(z, "z", (nb, L, nd), io, dev)
    _check(B, "B", (nb, L, ns), io, dev)
    _check(C, "C", (nb, L, ns), io, dev)
    _check(A, "A", (nd, ns), torch.float32, dev)
    _check(D, "D", (nd,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (nd,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (nb, L, nd), io, dev)
    return nb, L, nd, ns, out


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the binding allocates an output or workspace the caller did not pass: on the stream
    the kernels run on, so that the caching allocator never hands the block to other work while those
    kernels may still use it."""
    import contextlib

    torch = _torch()
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def bimamba_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, flags: int = 0, workspace=None,
                     stream=None):
    """Full-sequence bidirectional scan; returns out ([batch, seqlen, d_inner], x's dtype)."""
    torch = _torch()
    lib = load()
    with _on(stream):
        nb, L, nd, ns, out = _common(x, dt, A, B, C, D, z, dt_bias, out)
        need = int(lib.bimamba_scan_fwd_workspace_bytes(nb, L, nd, ns))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib.bimamba_scan_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                              _ptr(out), nb, L, nd, ns, _io_dtype(x), flags, _ptr(workspace),
                              _nbytes(workspace, x.device), _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_scan_fwd")
    return out


def bimamba_scan_fwd_noalloc(x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, flags: int = 0, stream=None):
    """bimamba_scan_fwd with the library's fixed scratch buffer as its workspace (the C call allocates nothing;
    out is allocated here only when not passed).  Returns out."""
    lib = load()
    with _on(stream):
        nb, L, nd, ns, out = _common(x, dt, A, B, C, D, z, dt_bias, out)
    st = lib.bimamba_scan_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                      _ptr(out), nb, L, nd, ns, _io_dtype(x), flags, _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_scan_fwd_noalloc")
    return out


def bimamba_scan_fwd_untied(fwd, rev, out_f=None, out_r=None, flags: int = 0, workspace=None, stream=None):
    """Untied directions: fwd and rev are dicts with keys x, dt, A, B, C and optionally D, z, dt_bias (each
    direction's own tensors).  Returns (out_f, out_r): the forward layer's gated output and the reverse layer's."""
    torch = _torch()
    f = {k: fwd.get(k) for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")}
    r = {k: rev.get(k) for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")}
    lib = load()
    with _on(stream):
        nb, L, nd, ns, out_f = _common(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["z"], f["dt_bias"],
                                       out_f)
        shape_r = _common(r["x"], r["dt"], r["A"], r["B"], r["C"], r["D"], r["z"], r["dt_bias"], out_r)
        if shape_r[:4] != (nb, L, nd, ns) or r["x"].dtype != f["x"].dtype:
            raise ValueError("the two directions must have the same shapes and I/O dtype")
        out_r = shape_r[4]
        need = int(lib.bimamba_scan_fwd_workspace_bytes(nb, L, nd, ns))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=f["x"].device)
    ptrs = [_ptr(f[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")] + [_ptr(out_f)]
    ptrs += [_ptr(r[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "dt_bias")] + [_ptr(out_r)]
    st = lib.bimamba_scan_fwd_untied(*ptrs, nb, L, nd, ns, _io_dtype(f["x"]), flags, _ptr(workspace),
                                     _nbytes(workspace, f["x"].device), _stream(stream, f["x"].device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_scan_fwd_untied")
    return out_f, out_r


def bimamba_scan_fwd_stage(stage: int, x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, flags: int = 0,
                           workspace=None, stream=None):
    """One stage (0 summary, 1 carry, 2 output) of bimamba_scan_fwd; the caller keeps workspace and out across
    the three calls.  Returns out."""
    with _on(stream):
        nb, L, nd, ns, out = _common(x, dt, A, B, C, D, z, dt_bias, out)
    if workspace is None:
        raise ValueError("the staged entry point needs a caller-kept workspace")
    st = load().bimamba_scan_fwd_stage(int(stage), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                       _ptr(dt_bias), _ptr(out), nb, L, nd, ns, _io_dtype(x), flags, _ptr(workspace),
                                       _nbytes(workspace, x.device), _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, f"bimamba_scan_fwd_stage({stage})")
    return out


def bimamba_scan_block(x, dt, A, B, C, D=None, z=None, dt_bias=None, h_in=None, h_out=None, out=None,
                       flags: int = 0, workspace=None, stream=None):
    """One block of block-cache decoding; returns out.  h_out (fp32 [batch, d_inner, d_state]) receives the
    forward state after the block when given (it may be the same tensor as h_in)."""
    torch = _torch()
    lib = load()
    with _on(stream):
        nb, L, nd, ns, out = _common(x, dt, A, B, C, D, z, dt_bias, out)
        _check(h_in, "h_in", (nb, nd, ns), torch.float32, x.device)
        _check(h_out, "h_out", (nb, nd, ns), torch.float32, x.device)
        need = int(lib.bimamba_scan_block_workspace_bytes(nb, L, nd, ns))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = _nbytes(workspace, x.device)
    st = lib.bimamba_scan_block(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                                _ptr(h_in), _ptr(h_out), _ptr(out), nb, L, nd, ns, _io_dtype(x), flags,
                                _ptr(workspace), wbytes, _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_scan_block")
    return out


def bimamba_ssd_fwd_workspace_bytes(batch: int, seqlen: int, nheads: int, headdim: int, d_state: int) -> int:
    return int(load().bimamba_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state))


def _ssd_common(x, dt, A, B, C, D, z, dt_bias, out):
    torch = _torch()
    if x.dim() != 3 or A.dim() != 1:
        raise ValueError("x must be [batch, seqlen, nheads*headdim] and A [nheads]")
    nb, L, nc = x.shape
    nh = A.shape[0]
    if nh == 0 or nc % nh:
        raise ValueError("the channel count must be a multiple of the head count")
    hp = nc // nh
    ns = B.shape[-1] if B.dim() == 3 else -1
    io = x.dtype
    dev = x.device
    _check(x, "x", (nb, L, nc), io, dev)
    _check(dt, "dt", (nb, L, nh), io, dev)
    _check(z, "z", (nb, L, nc), io, dev)
    _check(B, "B", (nb, L, ns), io, dev)
    _check(C, "C", (nb, L, ns), io, dev)
    _check(A, "A", (nh,), torch.float32, dev)
    _check(D, "D", (nh,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (nh,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (nb, L, nc), io, dev)
    return nb, L, nh, hp, ns, out


def bimamba_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, flags: int = 0, workspace=None,
                    stream=None):
    """Bidirectional Mamba-2 (SSD) scan over heads; returns out ([batch, seqlen, nheads*headdim], bf16).
    dt is [batch, seqlen, nheads]; A, D, dt_bias are [nheads] fp32."""
    torch = _torch()
    lib = load()
    with _on(stream):
        nb, L, nh, hp, ns, out = _ssd_common(x, dt, A, B, C, D, z, dt_bias, out)
        need = int(lib.bimamba_ssd_fwd_workspace_bytes(nb, L, nh, hp, ns))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib.bimamba_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                             _ptr(out), nb, L, nh, hp, ns, _io_dtype(x), flags, _ptr(workspace),
                             _nbytes(workspace, x.device), _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_ssd_fwd")
    return out


def bimamba_ssd_fwd_stage(stage: int, x, dt, A, B, C, D=None, z=None, dt_bias=None, out=None, flags: int = 0,
                          workspace=None, stream=None):
    """One stage (0 B/C tiles, 1 summaries, 2 carry, 3 output) of bimamba_ssd_fwd with a caller-kept workspace."""
    with _on(stream):
        nb, L, nh, hp, ns, out = _ssd_common(x, dt, A, B, C, D, z, dt_bias, out)
    if workspace is None:
        raise ValueError("the staged entry point needs a caller-kept workspace")
    st = load().bimamba_ssd_fwd_stage(int(stage), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(dt_bias), _ptr(out), nb, L, nh, hp, ns, _io_dtype(x), flags,
                                      _ptr(workspace), _nbytes(workspace, x.device), _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, f"bimamba_ssd_fwd_stage({stage})")
    return out


def bimamba_ssd_block_workspace_bytes(batch: int, block_len: int, nheads: int, headdim: int, d_state: int) -> int:
    return int(load().bimamba_ssd_block_workspace_bytes(batch, block_len, nheads, headdim, d_state))


def bimamba_ssd_block(x, dt, A, B, C, D=None, z=None, dt_bias=None, h_in=None, h_out=None, out=None,
                      flags: int = 0, workspace=None, stream=None):
    """One block of block-cache decoding with Mamba-2 heads; returns out.  h_in / h_out are fp32
    [batch, nheads, headdim, d_state] (h_out may be h_in): the cached forward state before and after the block."""
    torch = _torch()
    lib = load()
    with _on(stream):
        nb, L, nh, hp, ns, out = _ssd_common(x, dt, A, B, C, D, z, dt_bias, out)
        _check(h_in, "h_in", (nb, nh, hp, ns), torch.float32, x.device)
        _check(h_out, "h_out", (nb, nh, hp, ns), torch.float32, x.device)
        need = int(lib.bimamba_ssd_block_workspace_bytes(nb, L, nh, hp, ns))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib.bimamba_ssd_block(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                               _ptr(h_in), _ptr(h_out), _ptr(out), nb, L, nh, hp, ns, _io_dtype(x), flags,
                               _ptr(workspace), _nbytes(workspace, x.device), _stream(stream, x.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_ssd_block")
    return out


_LAYER_KEYS = ("xbc", "cw", "cb", "dt", "A", "D", "z", "dt_bias")


def bimamba_ssd_conv_untied(fwd=None, rev=None, out_f=None, out_r=None, flags: int = 0, d_state: int = 128,
                            workspace=None, stream=None):
    """Mamba-2 layers with untied directions, each with its short convolution.  fwd and rev are dicts with keys
    xbc ([batch, seqlen, H*P + 2*d_state] bf16), dt ([batch, seqlen, H]), A ([H]) and optionally cw
    ([H*P + 2*d_state, 4] fp32; None: no convolution), cb, D, dt_bias, z; either may be None to skip that layer.
    Returns (out_f, out_r), None for a skipped layer."""
    torch = _torch()
    sets = []
    with _on(stream):
        shape = None
        for d, o in ((fwd, out_f), (rev, out_r)):
            if d is None:
                sets.append(None)
                continue
            t = {k: d.get(k) for k in _LAYER_KEYS}
            xbc, A = t["xbc"], t["A"]
            if xbc.dim() != 3 or A.dim() != 1:
                raise ValueError("xbc must be [batch, seqlen, channels] and A [nheads]")
            nb, L, xs = xbc.shape
            nh = A.shape[0]
            hp = xs - 2 * d_state
            if nh == 0 or hp <= 0 or hp % nh:
                raise ValueError("xbc's channels must be nheads * headdim + 2 * d_state")
            if shape is not None and shape != (nb, L, xs, nh):
                raise ValueError("the two layers must have the same shapes")
            shape = (nb, L, xs, nh)
            dev, io = xbc.device, xbc.dtype
            _check(xbc, "xbc", (nb, L, xs), io, dev)
            _check(t["dt"], "dt", (nb, L, nh), io, dev)
            _check(t["z"], "z", (nb, L, hp), io, dev)
            for k in ("A", "D", "dt_bias"):
                _check(t[k], k, (nh,), torch.float32, dev)
            _check(t["cw"], "cw", (xs, 4), torch.float32, dev)
            _check(t["cb"], "cb", (xs,), torch.float32, dev)
            if o is None:
                o = torch.empty((nb, L, hp), dtype=io, device=dev)
            _check(o, "out", (nb, L, hp), io, dev)
            t["out"] = o
            sets.append(t)
        if shape is None:
            raise ValueError("at least one of fwd, rev is required")
        nb, L, xs, nh = shape
        hp = xs - 2 * d_state
        lib = load()
        if workspace is None:
            need = int(lib.bimamba_ssd_fwd_workspace_bytes(nb, L, nh, hp // nh, d_state))
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=next(t for t in sets if t)["xbc"].device)
    ptrs = []
    for t in sets:
        ptrs += [None] * 9 if t is None else [_ptr(t[k]) for k in _LAYER_KEYS + ("out",)]
    first = next(t for t in sets if t)
    dev = first["xbc"].device
    st = lib.bimamba_ssd_conv_untied(*ptrs, nb, L, nh, hp // nh, d_state, 4, _io_dtype(first["xbc"]), flags,
                                     _ptr(workspace), _nbytes(workspace, dev), _stream(stream, dev))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_ssd_conv_untied")
    return tuple(None if t is None else t["out"] for t in sets)


def _conv_common(u, w_f, b_f, w_r, b_r, out_f, out_r):
    torch = _torch()
    if u.dim() != 3:
        raise ValueError("u must be [batch, seqlen, channels]")
    nb, L, nc = u.shape
    if w_f is None and w_r is None:
        raise ValueError("at least one direction's filter is required")
    K = (w_f if w_f is not None else w_r).shape[-1]
    dev = u.device
    _check(u, "u", (nb, L, nc), u.dtype, dev)
    for name, t, shape in (("w_f", w_f, (nc, K)), ("w_r", w_r, (nc, K)), ("b_f", b_f, (nc,)), ("b_r", b_r, (nc,))):
        _check(t, name, shape, torch.float32, dev)
    if w_f is not None and out_f is None:
        out_f = torch.empty_like(u)
    if w_r is not None and out_r is None:
        out_r = torch.empty_like(u)
    _check(out_f, "out_f", (nb, L, nc), u.dtype, dev)
    _check(out_r, "out_r", (nb, L, nc), u.dtype, dev)
    return nb, L, nc, K, (out_f if w_f is not None else None), (out_r if w_r is not None else None)


def bimamba_conv1d_bidir(u, w_f=None, b_f=None, w_r=None, b_r=None, out_f=None, out_r=None, flags: int = 0,
                         stream=None):
    """Causal (w_f) and anti-causal (w_r) depthwise convolution of u with SiLU; returns (out_f, out_r), None for a
    direction whose filter is None."""
    with _on(stream):
        nb, L, nc, K, out_f, out_r = _conv_common(u, w_f, b_f, w_r, b_r, out_f, out_r)
    st = load().bimamba_conv1d_bidir(_ptr(u), _ptr(w_f), _ptr(b_f), _ptr(w_r), _ptr(b_r), _ptr(out_f), _ptr(out_r),
                                     nb, L, nc, K, _io_dtype(u), flags, _stream(stream, u.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_conv1d_bidir")
    return out_f, out_r


def bimamba_conv1d_block(u, w_f=None, b_f=None, w_r=None, b_r=None, cache_in=None, cache_out=None, out_f=None,
                         out_r=None, flags: int = 0, stream=None):
    """One block of block decoding: the causal filter continues from cache_in ([batch, 3, channels], u's dtype;
    None = zeros), the anti-causal one stops at the block end; cache_out (may be cache_in) receives the last 3
    tokens.  Returns (out_f, out_r)."""
    with _on(stream):
        nb, L, nc, K, out_f, out_r = _conv_common(u, w_f, b_f, w_r, b_r, out_f, out_r)
    _check(cache_in, "cache_in", (nb, K - 1, nc), u.dtype, u.device)
    _check(cache_out, "cache_out", (nb, K - 1, nc), u.dtype, u.device)
    st = load().bimamba_conv1d_block(_ptr(u), _ptr(w_f), _ptr(b_f), _ptr(w_r), _ptr(b_r), _ptr(cache_in),
                                     _ptr(cache_out), _ptr(out_f), _ptr(out_r), nb, L, nc, K, _io_dtype(u), flags,
                                     _stream(stream, u.device))
    if st != BIMAMBA_OK:
        raise BimambaError(st, "bimamba_conv1d_block")
    return out_f, out_r
