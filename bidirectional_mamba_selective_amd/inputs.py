"""Seeded synthetic inputs for the bidirectional selective scan.

This module only draws random numbers and rounds them to the I/O dtype; it
holds none of the scan's arithmetic.  Both the HIP tests and the oracle's
tests take their inputs from here, so the two sides always see the same bits.

Recipe (shapes follow the 1.3B-layer workloads the library is measured on):
  parameters (seed 0):
    u_d        = exp(Uniform(ln 1e-3, ln 1e-1))     per channel
    dt_bias[d] = log(expm1(u_d))                    so that softplus(dt_bias) = u_d
    A[d, n]    = -(n + 1)                           (exact in fp32)
    D[d]       = 1
  activations (seed 1, one independent stream per tensor):
    x, z, B, C ~ N(0, 1);  dt ~ 0.5 * N(0, 1)
    drawn in fp32 and rounded once, round-to-nearest-even, to the I/O dtype.
Every tensor uses its own PCG64 stream keyed by (seed, tensor id), so a
tensor does not change when another one changes size.

Mamba-2 (SSD) workloads, at the 1.3B layer's shape (120 heads of 32 channels,
state size 128):
  parameters (seed 0), one scalar per head:
    A[h]       = -Uniform(1, 16)
    dt_bias[h] = log(expm1(u_h)),  u_h = exp(Uniform(ln 1e-3, ln 1e-1))
    D[h]       = 1
  activations (seed 1): x, z [B, L, H*P] and B, C [B, L, N] ~ N(0, 1);
    dt [B, L, H] ~ 0.5 * N(0, 1); rounded to the I/O dtype as above.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_TENSOR_IDS = {"x": 1, "dt": 2, "z": 3, "B": 4, "C": 5, "xbc": 6, "dt_bias": 11, "A_jitter": 12, "A_head": 13,
               "conv_w": 14, "conv_b": 15}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    io_dtype: str  # "f32" or "bf16"
    calls: int = 1
    block_len: int = 0  # > 0: block-cache sweep with blocks of this many tokens


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32", 1, 256, 64, 16, "f32"),
        Workload("layer_2k_bf16", 1, 2048, 4096, 16, "bf16"),
        Workload("long_64k_bf16", 1, 65536, 4096, 16, "bf16"),
        Workload("batched_8k_bf16", 8, 8192, 2048, 16, "bf16", calls=128),
        Workload("block_32k_bf16", 1, 32768, 4096, 16, "bf16", block_len=32),
    )
}


def _rng(seed: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS[tensor]])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they denote (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """Round fp32 values to the I/O dtype and return them as exact fp32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if io_dtype == "f32":
        return a
    if io_dtype == "bf16":
        return bf16_bits_to_f32(bf16_bits(a))
    raise ValueError(io_dtype)


def make_params(d_inner: int, d_state: int, seed: int = 0, a_jitter: float = 0.0):
    """A [D, N], D [D], dt_bias [D] as fp32 arrays.

    a_jitter > 0 multiplies A by (1 + a_jitter * U(-1, 1)) per entry, giving a
    matrix without the per-channel geometric structure of the default init.
    """
    u = np.exp(_rng(seed, "dt_bias").uniform(np.log(1e-3), np.log(1e-1), size=d_inner))
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    A = -np.tile(np.arange(1, d_state + 1, dtype=np.float32), (d_inner, 1))
    if a_jitter > 0.0:
        j = _rng(seed, "A_jitter").uniform(-1.0, 1.0, size=A.shape).astype(np.float32)
        A = (A * (np.float32(1.0) + np.float32(a_jitter) * j)).astype(np.float32)
    D = np.ones(d_inner, dtype=np.float32)
    return np.ascontiguousarray(A), D, dt_bias


def normal(seed: int, tensor: str, shape, scale: float = 1.0, io_dtype: str = "f32") -> np.ndarray:
    """One seeded N(0, scale^2) tensor, rounded to io_dtype, returned as fp32."""
    a = _rng(seed, tensor).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return round_to(a, io_dtype)


def make_activations(batch: int, seqlen: int, d_inner: int, d_state: int, io_dtype: str, seed: int = 1,
                     xz_seed: int | None = None):
    """x, dt, z [B, L, D] and B, C [B, L, N] as fp32 arrays exact in io_dtype.

    xz_seed, when given, draws x and z from that seed instead (fresh
    activations per denoising call with dt, B, C held fixed).
    """
    s_xz = seed if xz_seed is None else xz_seed
    act = {
        "x": normal(s_xz, "x", (batch, seqlen, d_inner), 1.0, io_dtype),
        "dt": normal(seed, "dt", (batch, seqlen, d_inner), 0.5, io_dtype),
        "z": normal(s_xz, "z", (batch, seqlen, d_inner), 1.0, io_dtype),
        "B": normal(seed, "B", (batch, seqlen, d_state), 1.0, io_dtype),
        "C": normal(seed, "C", (batch, seqlen, d_state), 1.0, io_dtype),
    }
    return act


def make_workload_inputs(w: Workload, seed: int = 1, xz_seed: int | None = None, a_jitter: float = 0.0):
    """Parameters and activations for one workload (fp32 arrays)."""
    A, D, dt_bias = make_params(w.d_inner, w.d_state, a_jitter=a_jitter)
    act = make_activations(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, seed=seed, xz_seed=xz_seed)
    act.update(A=A, D=D, dt_bias=dt_bias)
    return act


@dataclass(frozen=True)
class SSDWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    d_state: int
    io_dtype: str = "bf16"


SSD_WORKLOADS = {
    w.name: w
    for w in (
        SSDWorkload("ssd_layer_2k_bf16", 1, 2048, 120, 32, 128),
        SSDWorkload("ssd_long_64k_bf16", 1, 65536, 120, 32, 128),
    )
}


def make_ssd_params(nheads: int, seed: int = 0):
    """A, D, dt_bias [nheads] as fp32 arrays (one scalar per head)."""
    A = -_rng(seed, "A_head").uniform(1.0, 16.0, size=nheads).astype(np.float32)
    u = np.exp(_rng(seed, "dt_bias").uniform(np.log(1e-3), np.log(1e-1), size=nheads))
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    D = np.ones(nheads, dtype=np.float32)
    return np.ascontiguousarray(A), D, dt_bias


def make_ssd_activations(batch: int, seqlen: int, nheads: int, headdim: int, d_state: int, io_dtype: str,
                         seed: int = 1):
    """x, z [B, L, H*P], dt [B, L, H] and B, C [B, L, N] as fp32 arrays exact in io_dtype."""
    nc = nheads * headdim
    return {
        "x": normal(seed, "x", (batch, seqlen, nc), 1.0, io_dtype),
        "dt": normal(seed, "dt", (batch, seqlen, nheads), 0.5, io_dtype),
        "z": normal(seed, "z", (batch, seqlen, nc), 1.0, io_dtype),
        "B": normal(seed, "B", (batch, seqlen, d_state), 1.0, io_dtype),
        "C": normal(seed, "C", (batch, seqlen, d_state), 1.0, io_dtype),
    }


def make_ssd_inputs(w: SSDWorkload, seed: int = 1):
    """Parameters and activations for one SSD workload (fp32 arrays)."""
    A, D, dt_bias = make_ssd_params(w.nheads)
    act = make_ssd_activations(w.batch, w.seqlen, w.nheads, w.headdim, w.d_state, w.io_dtype, seed=seed)
    act.update(A=A, D=D, dt_bias=dt_bias)
    return act


def make_ssd_layer_inputs(batch: int, seqlen: int, nheads: int, headdim: int = 32, d_state: int = 128,
                          seed: int = 1, param_seed: int = 0):
    """One Mamba-2 layer's inputs with its short convolution (the xBC stream of the projection):
    xbc [B, L, H*P + 2N] ~ N(0, 1), dt [B, L, H] ~ 0.5 N(0, 1), z [B, L, H*P] ~ N(0, 1), all rounded to bf16;
    conv taps [H*P + 2N, 4] ~ 0.5 N(0, 1) and bias [H*P + 2N] ~ 0.1 N(0, 1) (fp32, as in the convolution's
    tests), and the SSD parameters A, D, dt_bias per head (make_ssd_params)."""
    xs = nheads * headdim + 2 * d_state
    A, D, dt_bias = make_ssd_params(nheads, seed=param_seed)
    return {
        "xbc": normal(seed, "xbc", (batch, seqlen, xs), 1.0, "bf16"),
        "dt": normal(seed, "dt", (batch, seqlen, nheads), 0.5, "bf16"),
        "z": normal(seed, "z", (batch, seqlen, nheads * headdim), 1.0, "bf16"),
        "cw": normal(param_seed, "conv_w", (xs, 4), 0.5, "f32"),
        "cb": normal(param_seed, "conv_b", (xs,), 0.1, "f32"),
        "A": A, "D": D, "dt_bias": dt_bias,
    }


def device_normals(shapes: dict, seed: int, io_dtype: str, device="cuda", scales: dict | None = None):
    """Seeded N(0, scale^2) tensors drawn on the device with torch's generator (one stream per
    call, tensors in the order given), each drawn in fp32, scaled and rounded once (round to
    nearest even) to io_dtype.  The same distributions as `normal`, for tensors of several GiB
    that would take minutes to draw on the host."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dtype = torch.bfloat16 if io_dtype == "bf16" else torch.float32
    out = {}
    for name, shape in shapes.items():
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        s = (scales or {}).get(name, 1.0)
        if s != 1.0:
            t.mul_(s)
        out[name] = t.to(dtype)
        del t
    return out
