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
    rel, abs, mag: every element satisfies |o - r| <= rel * |r| + mag * m + abs * rms(r), where m is the sum
          of the magnitudes of the terms that make up that element (passed to check; see ssd_magnitudes).
    """

    def __init__(self, norm, row, rel, abs_, mag=0.0):
        self.norm, self.row, self.rel, self.abs, self.mag = norm, row, rel, abs_, mag


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
    # Mamba-2 heads: bf16 output; the products take bf16 operands with fp32 accumulation.  Written out over
    # the tokens and states it sums, an output element is a sum of terms C_i[n] B_j[n] dt_j x_j times a decay
    # (plus the skip term), each of which reaches the output through at most three bf16 roundings of 2^-9
    # relative: its weighted operand (the decay-weighted C B^T row, or the weighted x of a state update),
    # the state's operand copy in a readout, and the reverse sweep's partial output between the sweeps.  So
    # |o - r| <= 2^-8 |r| (the output's rounding) + 3 * 2^-9 * m, m = the sum of the terms' magnitudes (the
    # oracle on |x|, |B|, |C|, |D|, times |SiLU(z)|), plus fp32 accumulation (1e-6 of the rms).  An error
    # relative to the magnitudes, not to the element: large outputs of a long sequence (|r| ~ 20-80 rms) made
    # of terms several times larger reach 0.2-0.7 of 2^-8 m (measured over all 251 million outputs at
    # L = 65536).  Normwise 1.7e-3 - 2.1e-3; single tokens' rows up to ~4.4 % of the output's rms.
    "ssd": Bar(2e-2, 1e-1, _BF16_ROUND * 1.01, 1e-6, mag=3 * 2.0 ** -9),
    # the fp32 cache of the chunked Mamba-2 path: the same terms without the output rounding
    "ssd_state": Bar(1e-2, 1e-2, 1e-6, 1e-6, mag=3 * 2.0 ** -9),
    # two Mamba-2 results of the HIP path computed by different kernels: both errors, each within the "ssd" bound
    "ssd_pair": Bar(2e-2, 1e-1, 2 * _BF16_ROUND * 1.01, 2e-6, mag=6 * 2.0 ** -9),
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


def check(got, want, kind, tag="", quiet=False, mag=None):
    """Assert every bar of BARS[kind] (kind may also be a Bar) for got against want (fp64 arrays of one
    shape, rows along the last axis); mag, of the same shape, is required by bars with a magnitude term.
    Returns the measured figures; quiet leaves out the log line."""
    b = kind if isinstance(kind, Bar) else BARS[kind]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{tag}: shape {got.shape} != {want.shape}"
    assert not b.mag or (mag is not None and np.shape(mag) == want.shape), f"{tag}: the bar needs the magnitudes"
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
    if b.mag:
        allow = allow + b.mag * np.asarray(mag, dtype=np.float64)
    elem = float(np.max(np.abs(diff) / np.maximum(allow, 1e-300))) if want.size else 0.0
    res = {"norm": norm, "row": row, "elem": elem}
    if not quiet:
        say(f"{tag}: normwise {norm:.3e} (bar {b.norm:.0e}), worst row {row:.3e} (bar {b.row:.0e}), "
            f"worst element at {elem:.3f} of its bound")
    assert norm <= b.norm, f"{tag}: normwise rel err {norm:.3e} > {b.norm}"
    assert row <= b.row, f"{tag}: worst row rel err {row:.3e} > {b.row}"
    assert elem <= 1.0, (f"{tag}: an element exceeds |o-r| <= {b.rel:.2e}|r| + {b.abs:.0e} rms"
                         + (f" + {b.mag:.2e} m" if b.mag else "") + f" (x{elem:.2f})")
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
            for chan, part in pool.imap_unordered(_shard_call, np.array_split(np.arange(nchan), min(nchan, 4 * nw))):
                out[..., chan] = part
    finally:
        _SHARD.clear()
    return out


def ssd_magnitudes(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None, *, gate=True, fwd=True, rev=True):
    """For each Mamba-2 output element (and, with h0, each element of the new cache), the sum of the magnitudes
    of the terms it is made of: the oracle on |x|, |B|, |C|, |D| (and |h0|) without the gate (every decay and
    step size is positive), times |SiLU(z)| where the gate applies.  Returns mag_out, or (mag_out, mag_cache)
    when h0 is given."""
    import oracle

    ab = lambda a: None if a is None else np.abs(np.asarray(a, dtype=np.float64))  # noqa: E731
    if h0 is None:
        y = oracle.ssd_scan_fwd(ab(x), dt, A, ab(B), ab(C), ab(D), None, dt_bias, gate=False, fwd=fwd, rev=rev)
        hm = None
    else:
        y, hm = oracle.ssd_scan_block(ab(x), dt, A, ab(B), ab(C), ab(D), None, dt_bias, ab(h0), gate=False, fwd=fwd,
                                      rev=rev)
    if gate:
        y = y * np.abs(oracle.scan.silu(np.asarray(z, dtype=np.float64)))
    return y if h0 is None else (y, hm)


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
