#!/usr/bin/env python3
"""Throughput of the bidirectional selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_64k_bf16]

One step = one bimamba_scan_fwd call over the whole workload (summary, carry
and output kernels), inputs already resident in HBM.  W untimed steps, then K
timed steps bracketed by device synchronisations; one JSON line is printed.

Besides the headline tokens/s the line carries:
  roofline      the output kernel (the dominant one) against the VALU roofline,
                its duration measured live with HIP events on the stream the
                library launches on (staged entry point, same arguments);
  hbm           algorithmic bytes of the whole call / step time vs 8 TB/s;
  general_A, untied, ssd, conv
                the same shape off the geometric A path, with untied directions,
                the Mamba-2 heads and the short convolution (each with its own
                roofline where it has one);
  other_configs the batched workload (fresh x, z per call) and the block-variant
                sweep (--no-configs skips them);
  cpu_baseline  the fp64 oracle timed on this host on a bounded channel sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bidir selective-scan tokens/s + achieved HBM GB/s (% peak) at L=65536"
HBM_PEAK_GBS = 8000.0
# MI355X published fp32 vector peak; one fp32 FMA = 2 FLOP, one transcendental
# (v_exp_f32 / v_log_f32 / v_rcp_f32) issues at a quarter of the FMA rate and
# is counted as the 8 FLOP of the four FMA slots it occupies.
VALU_PEAK_TFLOPS = 157.3
FLOP_PER_ELEMENT_OUTPUT = 18  # per (token, channel, state): mul + exp(8) + mul + 2 fma(4) + 2 fma(4)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "k_output_long_64k_bf16_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "scan_kernels.hip")
SSD_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "ssd_kernels.hip")
CONV_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "conv_kernels.hip")
SSD_PROFILE = os.path.join(ROOT, "profiles", "k_ssd_long_64k_bf16_traffic.txt")
CONV_PROFILE = os.path.join(ROOT, "profiles", "k_conv_long_64k_bf16_traffic.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(batch, L, D, N, es):
    """Each input read once, out written once, A/D/dt_bias once per call."""
    per_token = 4 * D * es + 2 * N * es  # x, dt, z, out + B, C
    return batch * L * per_token + D * N * 4 + 2 * D * 4


def kernel_source_hash(path=None):
    return hashlib.sha256(open(path or KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def profiled_traffic(launch_elems=None, profile=None, source=None, key="hbm_bytes_per_dispatch"):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    profile = profile or PROFILE_TRAFFIC
    if not os.path.exists(profile):
        return None
    txt = open(profile).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash(source):
        return None
    return float(m_b.group(1))


def cpu_baseline(inp, L, D, nch):
    """The oracle as it stands on all L tokens of nch channels (exact for those channels:
    a channel's output depends on that channel and the shared B, C only), scaled to tokens/s of
    the full channel count.  numpy elementwise work runs on one thread."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    chan = np.linspace(0, D - 1, nch).astype(np.int64)
    sub = dict(x=inp["x"][:, :, chan], dt=inp["dt"][:, :, chan], z=inp["z"][:, :, chan], B=inp["B"], C=inp["C"],
               A=inp["A"][chan], D=inp["D"][chan], dt_bias=inp["dt_bias"][chan])
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx:
        with ctx:
            oracle.scan_fwd(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], sub["dt_bias"])
    else:
        oracle.scan_fwd(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], sub["dt_bias"])
    sec = time.perf_counter() - t0
    batch = inp["x"].shape[0]
    tok_s = batch * L / (sec * D / nch)
    return {"value": tok_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"all {batch}x{L} tokens of {nch} of {D} channels in {sec:.1f} s on 1 host thread, "
                      f"scaled by {D}/{nch} to the full channel count"}


def up_arr(a, w, torch, I, dev):
    """Host fp32 array (exact in the I/O dtype) -> device tensor of the workload's I/O dtype."""
    if w.io_dtype == "bf16":
        return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def bench_block(args, w, torch, bm, I, dev):
    """Block-decoding sweep: one bimamba_scan_block call per block of w.block_len tokens, the cached
    forward state carried in place from block to block.  A step is the whole sweep.  Reported: sweep
    tokens/s and us per block, both eager (one Python binding call per block, so host-side marshalling
    is included) and replayed from a HIP graph of the sweep's kernel launches (device-side cost)."""
    G = w.block_len
    nblk = w.seqlen // G
    log(f"workload {w.name}: batch {w.batch} L {w.seqlen} d_inner {w.d_inner} d_state {w.d_state} "
        f"{w.io_dtype}, {nblk} blocks of {G}")
    inp = I.make_workload_inputs(w)

    def up(k, io=True):
        a = inp[k]
        if io and w.io_dtype == "bf16":
            return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    full = {k: up(k) for k in ("x", "dt", "z", "B", "C")}
    A, Dv, bias = (up(k, False) for k in ("A", "D", "dt_bias"))
    # per-block contiguous inputs and outputs, resident in HBM before timing
    blk = [{k: full[k][:, b0:b0 + G].contiguous() for k in full} for b0 in range(0, w.seqlen, G)]
    outs = [torch.empty_like(b["x"]) for b in blk]
    h = torch.zeros(w.batch, w.d_inner, w.d_state, dtype=torch.float32, device=dev)
    need = bm.bimamba_scan_block_workspace_bytes(w.batch, G, w.d_inner, w.d_state)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if need else None
    stream = torch.cuda.current_stream(dev)

    def sweep():
        for b, o in zip(blk, outs):
            bm.bimamba_scan_block(b["x"], b["dt"], A, b["B"], b["C"], Dv, b["z"], bias, h_in=h, h_out=h, out=o,
                                  workspace=ws, stream=stream)

    for _ in range(args.warmup):
        h.zero_()
        sweep()
    torch.cuda.synchronize()
    t_eager = []
    for _ in range(args.steps):
        h.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sweep()
        torch.cuda.synchronize()
        t_eager.append(time.perf_counter() - t0)
    ref_out = torch.cat(outs, dim=1).clone()
    ref_h = h.clone()

    # the same sweep captured once as a graph (the library allocates nothing and issues no memsets)
    gstream = torch.cuda.Stream(dev)
    gstream.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(graph, stream=gstream):
            for b, o in zip(blk, outs):
                bm.bimamba_scan_block(b["x"], b["dt"], A, b["B"], b["C"], Dv, b["z"], bias, h_in=h, h_out=h,
                                      out=o, workspace=ws, stream=gstream)
    torch.cuda.synchronize()
    t_graph = []
    for r in range(max(3, args.steps)):
        h.zero_()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t_graph.append(time.perf_counter() - t0)
        same = torch.equal(torch.cat(outs, dim=1), ref_out) and torch.equal(h, ref_h)
        if not same:
            raise SystemExit(f"graph replay {r} differs from the eager sweep")
    # latency of one block step at other block lengths: 200 re-runs of one block from the same cache
    # (h_out = NULL, the denoising pattern before a commit), captured as a graph and replayed
    call_us = {}
    for Gc in (32, 64, 128):
        act = I.make_activations(w.batch, Gc, w.d_inner, w.d_state, w.io_dtype, seed=9)
        bl = {k: up_arr(act[k], w, torch, I, dev) for k in ("x", "dt", "z", "B", "C")}
        o = torch.empty_like(bl["x"])
        needc = bm.bimamba_scan_block_workspace_bytes(w.batch, Gc, w.d_inner, w.d_state)
        wsc = torch.empty(needc, dtype=torch.uint8, device=dev) if needc else None

        def one(s_):
            bm.bimamba_scan_block(bl["x"], bl["dt"], A, bl["B"], bl["C"], Dv, bl["z"], bias, h_in=h, h_out=None,
                                  out=o, workspace=wsc, stream=s_)

        one(stream)
        torch.cuda.synchronize()
        ref = o.clone()
        g2 = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream(dev)
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g2, stream=gs):
                for _ in range(200):
                    one(gs)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            o.zero_()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g2.replay()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
            if not torch.equal(o, ref):
                raise SystemExit(f"block G={Gc}: graph replay differs from the eager call")
        call_us[str(Gc)] = round(float(np.median(ts)) * 1e6 / 200, 2)
        log(f"block step G={Gc}: {call_us[str(Gc)]} us per call (graph of 200 re-runs)")

    tok = w.batch * w.seqlen
    te, tg = float(np.median(t_eager)), float(np.median(t_graph))
    log(f"sweep: eager {te * 1e3:.2f} ms, graph replay {tg * 1e3:.2f} ms (replays equal the eager result)")
    line = {
        "metric": "block-variant sweep tokens/s (one call per block, cached state carried)",
        "value": round(tok / tg, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tg * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io_dtype,
        "data": "synthetic (seeded N(0,1) activations, A[d,n]=-(n+1), D=1, log-uniform softplus(dt_bias))",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner,
                   "d_state": w.d_state, "block_len": G, "blocks": nblk, "io_dtype": w.io_dtype},
        "us_per_block_graph": round(tg * 1e6 / nblk, 2),
        "us_per_block_eager": round(te * 1e6 / nblk, 2),
        "tokens_per_s_eager": round(tok / te, 1),
        "workspace_bytes": need,
        "us_per_block_call_graph": call_us,
    }
    return line


def bench_batched(args, torch, bm, I, dev, stream, calls=16):
    """The batched workload as a denoising loop: `calls` calls with fresh x, z per call (drawn on the
    device outside the timed region, seed 1000 + call) and dt, B, C, A, D, dt_bias held fixed; each call
    timed with HIP events on the library's stream."""
    w = I.WORKLOADS["batched_8k_bf16"]
    log(f"batched workload {w.name}: batch {w.batch} L {w.seqlen} d_inner {w.d_inner} d_state {w.d_state}, "
        f"{calls} calls with fresh x, z")
    shp = (w.batch, w.seqlen, w.d_inner)
    fixed = I.device_normals({"dt": shp, "B": (w.batch, w.seqlen, w.d_state), "C": (w.batch, w.seqlen, w.d_state)},
                             seed=1, io_dtype=w.io_dtype, device=dev, scales={"dt": 0.5})
    A, Dv, bias = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
                   for a in I.make_params(w.d_inner, w.d_state))
    need = bm.bimamba_scan_fwd_workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    ms = []
    for s in range(calls + 2):
        xz = I.device_normals({"x": shp, "z": shp}, seed=1000 + s, io_dtype=w.io_dtype, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bm.bimamba_scan_fwd(xz["x"], fixed["dt"], A, fixed["B"], fixed["C"], Dv, xz["z"], bias, out=out, workspace=ws,
                            stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if s >= 2:  # the first two calls warm up
            ms.append(e0.elapsed_time(e1))
    m = float(np.mean(ms))
    log(f"batched: {m:.4f} ms per call (mean of {calls})")
    return {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner, "d_state": w.d_state,
            "calls": calls, "ms_per_call": round(m, 4), "tokens_per_s": round(w.batch * w.seqlen / (m * 1e-3), 1),
            "note": "fresh x, z per call drawn on the device outside the timed region; per-call HIP events"}


# matrix-core products per (64-token run, head) of the two SSD sweeps, and per run of the tiling kernel
SSD_Q, SSD_P, SSD_N = 64, 32, 128
SSD_FLOP_RSWEEP = 2 * SSD_Q * SSD_Q * SSD_P + 2 * SSD_Q * SSD_N * SSD_P + 2 * (2 * SSD_N * SSD_Q * SSD_P)
SSD_FLOP_FSWEEP = 2 * (2 * SSD_Q * SSD_N * SSD_P) + 2 * SSD_N * SSD_Q * SSD_P
SSD_FLOP_STAGE = 2 * SSD_Q * SSD_Q * SSD_N
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_ssd(args, torch, bm, I, dev, stream):
    """Mamba-2 (SSD) heads at the 1.3B layer's shape: one bimamba_ssd_fwd call per step."""
    w = I.SSD_WORKLOADS["ssd_long_64k_bf16"]
    log(f"ssd workload {w.name}: batch {w.batch} L {w.seqlen} heads {w.nheads} x {w.headdim} d_state {w.d_state}")
    inp = I.make_ssd_inputs(w)

    def up(a, io=True):
        if io:
            return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    x, dt, z, B, C = (up(inp[k]) for k in ("x", "dt", "z", "B", "C"))
    A, Dv, bias = (up(inp[k], False) for k in ("A", "D", "dt_bias"))
    del inp
    out = torch.empty_like(x)
    ws = torch.empty(bm.bimamba_ssd_fwd_workspace_bytes(w.batch, w.seqlen, w.nheads, w.headdim, w.d_state),
                     dtype=torch.uint8, device=dev)
    args_t = (x, dt, A, B, C, Dv, z, bias)

    def step():
        bm.bimamba_ssd_fwd(*args_t, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    names = ("k_ssd_stage", "k_ssd_rsweep", "k_ssd_carry", "k_ssd_fsweep")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        e = evs[s_]
        e[0].record(stream)
        for st in range(4):
            bm.bimamba_ssd_fwd_stage(st, *args_t, out=out, workspace=ws, stream=stream)
            e[st + 1].record(stream)
    torch.cuda.synchronize()
    per = {n: float(np.mean([evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]))
           for i, n in enumerate(names)}
    log(f"ssd: {ms:.4f} ms/call; per-kernel ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per.items()))
    runs = w.batch * ((w.seqlen + SSD_Q - 1) // SSD_Q)
    flop = {"k_ssd_rsweep": SSD_FLOP_RSWEEP * runs * w.nheads, "k_ssd_fsweep": SSD_FLOP_FSWEEP * runs * w.nheads,
            "k_ssd_stage": SSD_FLOP_STAGE * runs}
    dom = max(("k_ssd_rsweep", "k_ssd_fsweep"), key=lambda k: per[k])
    achieved = flop[dom] / (per[dom] * 1e-3) / 1e12
    tokens = w.batch * w.seqlen
    nc = w.nheads * w.headdim
    # HBM bytes the call must move: x twice (one per sweep), z once, out written twice and read once (the
    # reverse sweep's partial output), dt twice, B and C once; per run the tiling kernel writes C and B^T
    # (bf16) and C B^T (fp32), which the reverse sweep reads once and the forward sweep reads without C B^T
    tile = SSD_Q * SSD_N * 2
    io_bytes = (tokens * (nc * 2 * (2 + 1 + 3) + w.nheads * 2 * 2 + 2 * w.d_state * 2)
                + runs * (2 * tile + SSD_Q * SSD_Q * 4) * 2 + runs * 2 * tile)
    pages_flop = 2 * 2 * nc * w.d_state * tokens  # the paper's count: 2 d_inner d_state per token and direction
    del x, dt, z, B, C, out, ws
    block_us = ssd_block_latency(torch, bm, I, dev, w, A, Dv, bias)
    return {
        "workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
        "d_state": w.d_state, "io_dtype": "bf16", "state_dtype": "f32",
        "ms_per_call": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "kernels_ms": {k: round(v, 4) for k, v in per.items()},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "flop_per_launch": flop[dom],
                     "traffic": profiled_traffic(profile=SSD_PROFILE, source=SSD_SOURCE,
                                                 key=f"hbm_bytes_per_dispatch_{dom}")},
        "hbm": {"bytes_per_call": io_bytes, "achieved_gbs": round(io_bytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(io_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "scan_tflops_pages_count": round(pages_flop / (ms * 1e-3) / 1e12, 2),
        "block_step_us": block_us,
    }


def ssd_block_latency(torch, bm, I, dev, w, A, Dv, bias):
    """Block-cache decoding with the 120 heads: one bimamba_ssd_block step re-run 100 times from the same
    cache (h_out = NULL), captured as a graph and replayed; us per step at 32 and 64 tokens."""
    res = {}
    h = torch.zeros(1, w.nheads, w.headdim, w.d_state, dtype=torch.float32, device=dev)
    for G in (32, 64):
        act = I.make_ssd_activations(1, G, w.nheads, w.headdim, w.d_state, "bf16", seed=9)
        bl = {k: torch.from_numpy(I.bf16_bits(act[k]).view(np.int16)).view(torch.bfloat16).to(dev)
              for k in ("x", "dt", "z", "B", "C")}
        o = torch.empty_like(bl["x"])
        ws = torch.empty(bm.bimamba_ssd_block_workspace_bytes(1, G, w.nheads, w.headdim, w.d_state),
                         dtype=torch.uint8, device=dev)

        def one(s_):
            bm.bimamba_ssd_block(bl["x"], bl["dt"], A, bl["B"], bl["C"], Dv, bl["z"], bias, h_in=h, h_out=None,
                                 out=o, workspace=ws, stream=s_)

        gs = torch.cuda.Stream(dev)
        gs.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(gs):
            one(gs)
        torch.cuda.synchronize()
        ref = o.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for _ in range(100):
                    one(gs)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            o.zero_()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
            if not torch.equal(o, ref):
                raise SystemExit(f"ssd block G={G}: graph replay differs from the eager call")
        res[str(G)] = round(float(np.median(ts)) * 1e6 / 100, 2)
        log(f"ssd block step G={G}: {res[str(G)]} us per step (graph of 100 re-runs)")
    return res


def bench_conv(args, torch, bm, I, dev, stream):
    """The short causal / anti-causal convolution at the 1.3B layer's conv width (4096 channels), L = 65536, bf16:
    both directions from one read of the input."""
    L, C = 65536, 4096
    rng = np.random.default_rng(0)
    u = torch.from_numpy(I.bf16_bits(rng.standard_normal((1, L, C), dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16).to(dev)
    w_f, w_r = (torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32)).to(dev) for _ in range(2))
    b_f, b_r = (torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float32)).to(dev) for _ in range(2))
    out_f, out_r = torch.empty_like(u), torch.empty_like(u)

    def step():
        bm.bimamba_conv1d_bidir(u, w_f, b_f, w_r, b_r, out_f=out_f, out_r=out_r, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = L * C * 2 * 3  # u read once, both outputs written once
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"conv: {ms:.4f} ms/call, {gbs:.0f} GB/s")
    return {"workload": "conv_long_64k_bf16", "seq_len": L, "channels": C, "d_conv": 4, "io_dtype": "bf16",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(L / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "kernel": "k_conv", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                         "traffic": profiled_traffic(profile=CONV_PROFILE, source=CONV_SOURCE)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_64k_bf16")
    ap.add_argument("--cpu-channels", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ssd", action="store_true", help="skip the Mamba-2 (SSD) heads measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the batched and block-variant workloads reported beside the headline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the scan runs on a single MI355X and this build has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bidirectional_mamba_selective_amd as bm
    from bidirectional_mamba_selective_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bm.load()
    if w.block_len:
        print(json.dumps(bench_block(args, w, torch, bm, I, dev)), flush=True)
        return

    log(f"workload {w.name}: batch {w.batch} L {w.seqlen} d_inner {w.d_inner} d_state {w.d_state} {w.io_dtype}")
    t0 = time.perf_counter()
    inp = I.make_workload_inputs(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def up(k, io=True):
        a = inp[k]
        if io and w.io_dtype == "bf16":
            return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    x, dt, z, B, C = (up(k) for k in ("x", "dt", "z", "B", "C"))
    A, Dv, bias = (up(k, False) for k in ("A", "D", "dt_bias"))
    # the same workload with A moved off its per-channel geometric structure (general exponential path)
    A_gen = torch.from_numpy(I.make_params(w.d_inner, w.d_state, a_jitter=0.2)[0]).to(dev)
    out = torch.empty_like(x)
    need = bm.bimamba_scan_fwd_workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(a_mat=A):
        bm.bimamba_scan_fwd(x, dt, a_mat, B, C, Dv, z, bias, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_step_ev = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step wall, {ms_step_ev:.4f} ms/step events")

    # the general-A path on the same inputs (reported beside the headline)
    for _ in range(2):
        step(A_gen)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(A_gen)
    torch.cuda.synchronize()
    ms_step_gen = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"general A: {ms_step_gen:.4f} ms/step")

    # untied directions on the same shape: a second input and parameter set for the reverse layer
    act_r = I.make_activations(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, seed=2)
    A_r, D_r, bias_r = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
                        for a in I.make_params(w.d_inner, w.d_state, seed=1))
    rev_set = dict(x=up_arr(act_r["x"], w, torch, I, dev), dt=up_arr(act_r["dt"], w, torch, I, dev),
                   z=up_arr(act_r["z"], w, torch, I, dev), B=up_arr(act_r["B"], w, torch, I, dev),
                   C=up_arr(act_r["C"], w, torch, I, dev), A=A_r, D=D_r, dt_bias=bias_r)
    del act_r
    fwd_set = dict(x=x, dt=dt, z=z, B=B, C=C, A=A, D=Dv, dt_bias=bias)
    out_r = torch.empty_like(x)

    def step_untied():
        bm.bimamba_scan_fwd_untied(fwd_set, rev_set, out_f=out, out_r=out_r, workspace=ws, stream=stream)

    for _ in range(2):
        step_untied()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_untied()
    torch.cuda.synchronize()
    ms_step_untied = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"untied directions: {ms_step_untied:.4f} ms/step")

    # per-kernel attribution on the same stream: staged entry point, events between stages
    names = ("k_summary", "k_carry", "k_output")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        e = evs[s]
        e[0].record(stream)
        for st in range(3):
            bm.bimamba_scan_fwd_stage(st, x, dt, A, B, C, Dv, z, bias, out=out, workspace=ws, stream=stream)
            e[st + 1].record(stream)
    torch.cuda.synchronize()
    per = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}
    log("per-kernel ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per.items()))

    if args.calibrate_copy:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(buf)
        for _ in range(3):
            dst.copy_(buf)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB done")

    es = 2 if w.io_dtype == "bf16" else 4
    elems = w.batch * w.seqlen * w.d_inner * w.d_state
    tokens = w.batch * w.seqlen
    abytes = algorithmic_bytes(w.batch, w.seqlen, w.d_inner, w.d_state, es)
    t_out = per["k_output"] * 1e-3
    achieved = FLOP_PER_ELEMENT_OUTPUT * elems / t_out / 1e12
    traffic = profiled_traffic(elems) if w.name == "long_64k_bf16" else None
    roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / VALU_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "k_output (output pass; the workload's A takes its geometric body)",
                "kernel_ms": round(per["k_output"], 4)}
    hbm_gbs = abytes / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io_dtype if w.io_dtype != "f32" else "f32",
        "data": "synthetic (seeded N(0,1) activations, A[d,n]=-(n+1), D=1, log-uniform softplus(dt_bias))",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner,
                   "d_state": w.d_state, "io_dtype": w.io_dtype, "state_dtype": "f32"},
        "roofline": roofline,
        "hbm": {"algorithmic_bytes": abytes, "achieved_gbs": round(hbm_gbs, 1),
                "frac_of_peak": round(hbm_gbs / HBM_PEAK_GBS, 4), "peak_gbs": HBM_PEAK_GBS},
        "kernels_ms": {k: round(v, 4) for k, v in per.items()},
        "general_A": {"ms_per_step": round(ms_step_gen, 4), "tokens_per_s": round(tokens / (ms_step_gen * 1e-3), 1),
                      "note": "A[d,n] = -(n+1)*(1+0.2*U(-1,1)): no per-channel geometric structure, one exp per "
                              "(token, channel, state) in each pass"},
        "ms_per_step_events": round(ms_step_ev, 4),
        "untied": {"ms_per_step": round(ms_step_untied, 4),
                   "tokens_per_s": round(tokens / (ms_step_untied * 1e-3), 1),
                   "note": "each direction its own x, dt, B, C, z, A, D, dt_bias and its own gated output "
                           "(bimamba_scan_fwd_untied): a forward-only and a reverse-only pass, twice the "
                           "activation bytes and no shared abar"},
    }
    if not args.no_ssd:
        del x, dt, z, B, C, out, out_r, rev_set, fwd_set, ws
        torch.cuda.empty_cache()
        line["ssd"] = bench_ssd(args, torch, bm, I, dev, stream)
        torch.cuda.empty_cache()
        line["conv"] = bench_conv(args, torch, bm, I, dev, stream)
    if not args.no_configs and w.name == "long_64k_bf16":
        torch.cuda.empty_cache()
        other = {"batched_8k_bf16": bench_batched(args, torch, bm, I, dev, stream)}
        torch.cuda.empty_cache()
        bl = bench_block(argparse.Namespace(steps=3, warmup=1), I.WORKLOADS["block_32k_bf16"], torch, bm, I, dev)
        other["block_32k_bf16"] = {k: bl[k] for k in ("value", "unit", "ms_per_step", "us_per_block_graph",
                                                       "us_per_block_eager", "us_per_block_call_graph")}
        other["block_32k_bf16"]["metric"] = bl["metric"]
        line["other_configs"] = other
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_channels} channels")
        line["cpu_baseline"] = cpu_baseline(inp, w.seqlen, w.d_inner, min(args.cpu_channels, w.d_inner))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
