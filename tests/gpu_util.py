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
