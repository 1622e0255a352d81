"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI (ctypes binding), run the oracle on the same bits, compare."""
from __future__ import annotations

import sys
import time

import numpy as np

from bidirectional_mamba_selective_amd.inputs import bf16_bits


def say(msg: str) -> None:
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def torch_mod():
    import torch

    return torch


def to_dev(a, io_dtype, dev="cuda"):
    torch = torch_mod()
    if a is None:
        return None
    if io_dtype == "bf16":
        return torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def f32_dev(a, dev="cuda"):
    torch = torch_mod()
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_host64(t):
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want.ravel())
    num = np.linalg.norm((got - want).ravel())
    return float(num / den) if den > 0 else float(num)


def tol_for(io_dtype):
    # parity bars: normwise relative error <= 2e-2 with bf16 I/O, <= 1e-4 with fp32 I/O
    return 2e-2 if io_dtype == "bf16" else 1e-4


class Bar:
    """Parity bars for one kind of result.

    norm: ||o - r|| / ||r|| over the whole compared tensor (the target's tolerance);
    row:  the same ratio for every row (the last axis: the compared channels of one token, or the states of
          one channel), with ||r_row|| floored at abs/row (at least 5 %) of the rms row norm, so that rows the
          gate or the data make nearly zero are held to the absolute level the elementwise bound allows;
    rel, abs: every element satisfies |o - r| <= rel * |r| + abs * rms(r).
    """

    def __init__(self, norm, row, rel, abs_):
        self.norm, self.row, self.rel, self.abs = norm, row, rel, abs_


# bf16 output: the kernel's fp32 result y is rounded to nearest even, |o - y| <= 2^-8 |y| (half an ulp of an
# 8-bit significand), so |o - r| <= 2^-8 |r| + (1 + 2^-8) |y - r|; the fp32 arithmetic before the rounding
# (|y - r|) is covered by the absolute term.
_BF16_ROUND = 2.0 ** -8
BARS = {
    # Per-channel S6 scan, fp32 I/O.  The target's 1e-4 normwise and per token; elementwise 1e-4 relative
    # plus 3e-5 of the rms for elements that cancellation makes small: the sums over tokens, states and
    # directions carry fp32 rounding of ~1e-6 of the rms, and with dt_bias 60 below its recipe range the
    # step size e^v comes from an exponential of an argument near -94, whose fp32 rounding alone gives
    # delta up to ~4e-6 relative error (measured up to 1.0e-5 of the rms on one element in 77k).
    "f32": Bar(1e-4, 1e-4, 1e-4, 3e-5),
    # bf16 I/O: the target's 2e-2 normwise and per token; elementwise the rounding bound above plus 2e-4 rms
    "bf16": Bar(2e-2, 2e-2, _BF16_ROUND * 1.01, 2e-4),
    # the short convolution in fp32: four products and a SiLU per output
    "conv_f32": Bar(1e-5, 1e-5, 1e-5, 1e-6),
    # fp32 states (the block cache of the S6 scan): 2e-5 relative plus 3e-6 of the rms; the cache after
    # hundreds of tokens is a sum of that many decayed fp32 terms (measured up to 1.2e-6 of the rms)
    "state": Bar(1e-5, 1e-5, 2e-5, 3e-6),
    # Mamba-2 heads: bf16 output; the products take bf16 operands with fp32 accumulation, so an output
    # element carries the rounding of its operands (2^-9 of each term of the intra-run and readout sums),
    # which is relative to the size of the terms, not of the element: normwise 1.7e-3 - 3e-3, single elements
    # up to ~6.4 % (one in 4 million) and single tokens' rows up to ~4.4 % of the output's rms
    "ssd": Bar(2e-2, 1e-1, _BF16_ROUND * 1.01, 8e-2),
    "ssd_state": Bar(1e-2, 1e-2, 1e-2, 2e-2),
    # Mamba-2 cache of the single-kernel block step, whose products take each fp32 operand as two bf16 values:
    # hi = bf16(v) within 2^-8 |v|, lo = bf16(v - hi) within 2^-8 |v - hi|, so each term of a 64-token
    # increment is carried to 2^-16 of its size; for N(0,1) operands the sum of the terms' magnitudes is about
    # 5x the rms of the sum, so an element's error stays under 2^-16 * 5 = 8e-5 of the rms (abs); normwise and
    # per row the errors are independent across terms, far below that (measured over 256 chained blocks:
    # 3.8e-6 normwise, 9.2e-6 per row, 3.4e-5 of the rms on single elements)
    "ssd_split_state": Bar(1e-5, 3e-5, 2e-5, 8e-5),
}


def bar_for(kind):
    return BARS[kind]


def check(got, want, kind, tag="", quiet=False):
    """Assert every bar of BARS[kind] (kind may also be a Bar) for got against want (fp64 arrays of one
    shape, rows along the last axis).  Returns the measured figures; quiet leaves out the log line."""
    b = kind if isinstance(kind, Bar) else BARS[kind]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{tag}: shape {got.shape} != {want.shape}"
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    diff = got - want
    den = np.linalg.norm(want.ravel())
    norm = float(np.linalg.norm(diff.ravel()) / den) if den > 0 else float(np.linalg.norm(diff.ravel()))
    w2 = want.reshape(-1, want.shape[-1]) if want.ndim > 1 else want.reshape(1, -1)
    d2 = diff.reshape(w2.shape)
    rn = np.linalg.norm(w2, axis=1)
    floor = max(0.05, b.abs / b.row) * float(np.sqrt(np.mean(rn ** 2))) if rn.size else 0.0
    floor = max(floor, 1e-300)
    row = float(np.max(np.linalg.norm(d2, axis=1) / np.maximum(rn, floor))) if rn.size else 0.0
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    allow = b.rel * np.abs(want) + b.abs * rms
    elem = float(np.max(np.abs(diff) / np.maximum(allow, 1e-300))) if want.size else 0.0
    res = {"norm": norm, "row": row, "elem": elem}
    if not quiet:
        say(f"{tag}: normwise {norm:.3e} (bar {b.norm:.0e}), worst row {row:.3e} (bar {b.row:.0e}), "
            f"worst element at {elem:.3f} of its bound")
    assert norm <= b.norm, f"{tag}: normwise rel err {norm:.3e} > {b.norm}"
    assert row <= b.row, f"{tag}: worst row rel err {row:.3e} > {b.row}"
    assert elem <= 1.0, f"{tag}: an element exceeds |o-r| <= {b.rel:.2e}|r| + {b.abs:.0e} rms (x{elem:.2f})"
    return res


# The inputs of oracle_sharded's worker processes: set before the workers are forked (they inherit them
# copy-on-write, run numpy only and touch no GPU) and cleared afterwards.
_SHARD = {}


def _shard_call(chan):
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        return chan, _SHARD["fn"](_SHARD["inp"], chan)


def oracle_sharded(fn, inp, nchan, out_shape, workers=8):
    """fn(inp, chan) -> the oracle's output on channels `chan` (the last axis), run over all nchan channels in
    shards by up to `workers` forked host processes.  Exact: a channel's output depends only on that channel
    and the shared B, C (the oracle pin on channel independence)."""
    import multiprocessing as mp
    import os

    nw = max(1, min(workers, len(os.sched_getaffinity(0))))
    out = np.empty(out_shape)
    _SHARD.clear()
    _SHARD.update(fn=fn, inp=inp)
    try:
        with mp.get_context("fork").Pool(nw) as pool:
            for chan, part in pool.imap_unordered(_shard_call, np.array_split(np.arange(nchan), 4 * nw)):
                out[..., chan] = part
    finally:
        _SHARD.clear()
    return out


def upload(inp, io_dtype):
    """Device tensors for one input dict of fp32 arrays (exact in io_dtype)."""
    dev = {}
    for k in ("x", "dt", "z", "B", "C"):
        dev[k] = to_dev(inp.get(k), io_dtype)
    for k in ("A", "D", "dt_bias"):
        dev[k] = f32_dev(inp.get(k))
    return dev


def run_fwd(dev, flags=0, use_D=True, use_bias=True, use_z=True):
    from bidirectional_mamba_selective_amd import bimamba_scan_fwd

    torch = torch_mod()
    out = bimamba_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"] if use_D else None,
                           dev["z"] if use_z else None, dev["dt_bias"] if use_bias else None, flags=flags)
    torch.cuda.synchronize()
    return out


def oracle_fwd(inp, chan=None, gate=True, fwd=True, rev=True, use_D=True, use_bias=True):
    import oracle

    def sel(k):
        a = inp[k]
        if chan is None:
            return a
        if k in ("x", "dt", "z"):
            return a[:, :, chan]
        if k == "A":
            return a[chan]
        if k in ("D", "dt_bias"):
            return a[chan]
        return a

    return oracle.scan_fwd(sel("x"), sel("dt"), sel("A"), sel("B"), sel("C"), sel("D") if use_D else None,
                           sel("z") if gate else None, sel("dt_bias") if use_bias else None, gate=gate, fwd=fwd,
                           rev=rev)
