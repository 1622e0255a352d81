#!/usr/bin/env python3
"""Throughput of the bidirectional selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_64k_bf16]

One step = one bimamba_scan_fwd call over the whole workload (summary, carry
and output kernels), inputs already resident in HBM.  W untimed steps (continued
until a quarter second of them has run, so that the shader clock has settled),
then K timed steps bracketed by device synchronisations; one JSON line is
printed.  The K steps timed after an idle second and W steps only are reported
beside them (ms_per_step_after_idle).

Besides the headline tokens/s the line carries:
  roofline      the output kernel (the dominant one) against the HBM roofline:
                the call's algorithmic bytes (each input read once, out written
                once) over that kernel's duration, measured live with HIP events
                on the stream the library launches on (staged entry point, same
                arguments), against 8 TB/s; traffic = the kernel's counter bytes;
  valu          the same kernel's VALU issue: measured instructions per element
                (committed counters) against the issue rate measured by the
                microbenchmarks;
  hbm           algorithmic bytes of the whole call / step time vs 8 TB/s;
  micro         HBM read and copy streams, FMA and v_exp_f32 issue rates, and the
                empty-kernel launch floor (graph replay) on this machine;
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
NOMINAL_CLOCK_GHZ = 2.4  # MI355X peak engine clock; 256 CUs of 4 SIMDs
N_SIMD = 1024
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "k_output_long_64k_bf16_traffic.txt")
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "k_output_long_64k_bf16_counters.txt")
MICRO_LIB = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "libbimamba_micro.so")
KERNEL_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "scan_kernels.hip")
SSD_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "ssd_kernels.hip")
CONV_SOURCE = os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", "conv_kernels.hip")
SSD_PROFILE = os.path.join(ROOT, "profiles", "k_ssd_long_64k_bf16_traffic.txt")
CONV_PROFILE = os.path.join(ROOT, "profiles", "k_conv_long_64k_bf16_traffic.txt")
SSDCONV_PROFILE = os.path.join(ROOT, "profiles", "k_ssd1_conv_long_64k_bf16_traffic.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The shader clock drops whenever the GPU idles and climbs back over the first 10-15 calls of the
# workload once work resumes (measured on MI355X at L = 65536: 1.86-2.15 ms per call right after half
# a second of idle, 1.61-1.66 ms once settled).  Each timed region below therefore follows W untimed
# steps continued until at least SETTLE_S seconds of them have run; the headline also reports the K
# steps timed after an idle second and W steps only (ms_per_step_after_idle).
SETTLE_S = 0.25


def warm(fn, steps, torch, seconds=SETTLE_S):
    """Run fn at least `steps` times and until `seconds` of them have run (synchronising every 8 calls so
    that the host does not run ahead of the GPU); returns the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while n < steps or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


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


def profiled_counters(kernel="k_output"):
    """VALU instructions per SIMD and lane operations per element of one kernel from the committed SQ
    counter summary, or None when it is missing or was taken on a different kernel source."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    txt = open(PROFILE_COUNTERS).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m_src or m_src.group(1) != kernel_source_hash():
        return None
    sec = txt.split(kernel + "<", 1)
    if len(sec) < 2:
        return None
    m = re.search(r"VALU instructions per SIMD:\s*([0-9.eE+]+); lane operations per \(token, channel, state\):"
                  r"\s*([0-9.]+)", sec[1])
    return None if not m else {"instructions_per_simd": float(m.group(1)), "lane_ops_per_element": float(m.group(2))}


# The oracle's inputs for the all-cores CPU baseline, set before the worker processes are forked (they
# inherit them copy-on-write) and cleared afterwards.
_CPU_SHARED = {}


def _oracle_channels(chan):
    import oracle
    from threadpoolctl import threadpool_limits

    s = _CPU_SHARED
    with threadpool_limits(1):
        oracle.scan_fwd(s["x"][:, :, chan], s["dt"][:, :, chan], s["A"][chan], s["B"], s["C"], s["D"][chan],
                        s["z"][:, :, chan], s["dt_bias"][chan])
    return len(chan)


def cpu_baseline(inp, L, D, nch1, workers):
    """The oracle as it stands, timed on this host: (1) on one thread over all L tokens of nch1 channels,
    scaled to the full channel count; (2) over the whole workload (every token and channel), its channels
    split evenly across `workers` processes, one thread each.  Both are exact for the channels they run: a
    channel's output depends only on that channel and the shared B, C.  The all-cores figure is the value."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    batch = inp["x"].shape[0]
    chan = np.linspace(0, D - 1, nch1).astype(np.int64)
    _CPU_SHARED.clear()
    _CPU_SHARED.update(inp)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        _oracle_channels(chan)
        sec1 = time.perf_counter() - t0
    tok_s1 = batch * L / (sec1 * D / nch1)
    shards = np.array_split(np.arange(D, dtype=np.int64), workers)
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(len, [[0]] * workers)  # the workers are up before the clock starts
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_channels, shards, chunksize=1))
        secn = time.perf_counter() - t0
    _CPU_SHARED.clear()
    assert done == D
    return {"value": round(batch * L / secn, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"the whole workload ({batch}x{L} tokens, {D} channels) in {secn:.1f} s, its channels split "
                      f"over {workers} processes of one thread each; one thread: {nch1} of {D} channels in "
                      f"{sec1:.1f} s, scaled by {D}/{nch1} to {tok_s1:.0f} tokens/s",
            "value_1core": round(tok_s1, 1)}


def host_workers():
    """Worker processes for the all-cores CPU baseline: the host cores this process may run on, at most 16
    (a GPU machine's CPU share per GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def bench_micro(torch, dev, stream):
    """Microbenchmarks on this machine, each timed with HIP events on `stream` (median of 5): HBM read-only and
    copy streams over 4 GiB and 2 GiB, the issue rate of independent fp32 FMAs and of v_exp_f32 at 1 to 8
    wavefronts per SIMD, FMAs with SGPR and DPP-broadcast operands, and an empty kernel's launch floor replayed from a graph (one 64-lane workgroup,
    and the block step's grid of 256 workgroups of 512 threads)."""
    import ctypes

    if not os.path.exists(MICRO_LIB):
        raise RuntimeError(f"{MICRO_LIB} is missing: build it with `python -m bidirectional_mamba_selective_amd.build`")
    lib = ctypes.CDLL(MICRO_LIB)
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.micro_read.argtypes = [vp, sz, vp, vp]
    lib.micro_copy.argtypes = [vp, vp, sz, vp]
    lib.micro_fma.argtypes = [vp, ci, ci, vp, vp]
    lib.micro_exp.argtypes = [vp, ci, ci, vp]
    lib.micro_fma_operand.argtypes = [vp, ci, ci, ci, vp]
    lib.micro_empty.argtypes = [ci, ci, vp]
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps=5):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"micro kernel launch failed: {st}")
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts[1:]))

    res = {}
    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    t = timed(lambda: lib.micro_read(ctypes.c_void_p(src.data_ptr()), src.numel(), ctypes.c_void_p(sink.data_ptr()),
                                     sp))
    res["hbm_read_gbs"] = round(src.numel() / t / 1e9, 1)
    half = src.numel() // 2
    t = timed(lambda: lib.micro_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(src.data_ptr() + half), half,
                                     sp))
    res["hbm_copy_gbs"] = round(2 * half / t / 1e9, 1)  # bytes read + bytes written
    del src
    clk = torch.zeros(8192, dtype=torch.int64, device=dev)
    # the shader clock under a full FMA load at 4 wavefronts per SIMD (the scans' occupancy)
    lib.micro_fma(ctypes.c_void_p(sink.data_ptr()), 1024, 4, ctypes.c_void_p(clk.data_ptr()), sp)
    torch.cuda.synchronize()
    c = clk.cpu().numpy().reshape(-1, 2)
    ghz = float(np.median(c[:, 0] / np.maximum(c[:, 1], 1))) * 0.1
    res["clock_ghz_under_fma_load"] = round(ghz, 3)
    fma, ex = {}, {}
    for w in (1, 2, 4, 8):
        iters = 1024
        t = timed(lambda: lib.micro_fma(ctypes.c_void_p(sink.data_ptr()), iters, w, ctypes.c_void_p(clk.data_ptr()),
                                        sp))
        rate = N_SIMD * w * 64 * 64 * iters / t  # lane-FMAs per second (64 per thread and iteration)
        fma[str(w)] = round(rate / (256 * ghz * 1e9), 1)  # per clock and CU at the measured clock
        t = timed(lambda: lib.micro_exp(ctypes.c_void_p(sink.data_ptr()), 1024, w, sp))
        ex[str(w)] = round(N_SIMD * w * 64 * 8 * 1024 / t / (256 * ghz * 1e9), 1)
    res["fma_lanes_per_clk_per_cu"] = fma
    res["exp_lanes_per_clk_per_cu"] = ex
    # clocks per wave64 FMA instruction and SIMD at 4 wavefronts per SIMD (the scan kernels' occupancy)
    res["fma_clk_per_instruction_4waves"] = round(64 * 4 / fma["4"], 3)
    # the same at 8 wavefronts per SIMD
    res["fma_clk_per_instruction_8waves"] = round(64 * 4 / fma["8"], 3)
    # clocks per wavefront FMA instruction and SIMD by the kind of the multiplier operand, 32 chains in one
    # harness: lane-varying VGPR, wave-uniform SGPR in every FMA or in every other one, a VGPR read through the
    # DPP row broadcast (row_newbcast), at 4 and 8 wavefronts per SIMD
    sg = {}
    for w in (4, 8):
        row = {}
        for mode, name in ((0, "vgpr"), (1, "sgpr_every_fma"), (2, "sgpr_every_other_fma"), (3, "dpp_row_bcast")):
            t = timed(lambda: lib.micro_fma_operand(ctypes.c_void_p(sink.data_ptr()), 2048, w, mode, sp))
            row[name] = round(t * ghz * 1e9 / (w * 64 * 2048), 3)
        sg[str(w)] = row
    res["fma_operand_clk_per_instruction"] = sg

    floor = {}
    for groups, threads in ((1, 64), (256, 512)):
        gs = torch.cuda.Stream(dev)
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for _ in range(200):
                    lib.micro_empty(groups, threads, ctypes.c_void_p(gs.cuda_stream))
        torch.cuda.synchronize()
        ts = []
        for _ in range(4):
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        floor[f"{groups}x{threads}"] = round(float(np.median(ts[1:])) * 1e6 / 200, 2)
    res["empty_kernel_graph_us"] = floor
    log(f"micro: read {res['hbm_read_gbs']} GB/s, copy {res['hbm_copy_gbs']} GB/s, fma lanes/clk/CU {fma}, "
        f"exp {ex}, fma clk/instr by operand {sg}, empty-kernel graph floor {floor} us")
    return res


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
    warm(graph.replay, 3, torch)
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
        warm(g2.replay, 3, torch)
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


def bench_batched(args, torch, bm, I, dev, stream, calls=128):
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
    xz = I.device_normals({"x": shp, "z": shp}, seed=999, io_dtype=w.io_dtype, device=dev)
    warm(lambda: bm.bimamba_scan_fwd(xz["x"], fixed["dt"], A, fixed["B"], fixed["C"], Dv, xz["z"], bias, out=out,
                                     workspace=ws, stream=stream), 2, torch)
    del xz
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
    tot = float(np.sum(ms))
    log(f"batched: {calls} calls, {tot:.2f} ms in all, {m:.4f} ms per call")
    return {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner, "d_state": w.d_state,
            "calls": calls, "ms_all_calls": round(tot, 3), "ms_per_call": round(m, 4),
            "tokens_per_s": round(calls * w.batch * w.seqlen / (tot * 1e-3), 1),
            "note": "the workload's 128 denoising calls, fresh x, z per call drawn on the device outside the timed "
                    "region; per-call HIP events summed"}


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

    warm(step, args.warmup, torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    names = ("k_ssd_stage", "k_ssd_rsweep", "k_ssd_carry", "k_ssd_fsweep")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    warm(step, args.warmup, torch)
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
    dom = max(per, key=lambda k: per[k])
    tokens = w.batch * w.seqlen
    nc = w.nheads * w.headdim
    # algorithmic bytes: x, z read once, out written once, dt, B, C read once (A, D, dt_bias: 3 floats per head)
    io_bytes = tokens * (3 * nc * 2 + w.nheads * 2 + 2 * w.d_state * 2) + 3 * w.nheads * 4
    pages_flop = 2 * 2 * nc * w.d_state * tokens  # the paper's count: 2 d_inner d_state per token and direction
    gbs_dom = io_bytes / (per[dom] * 1e-3) / 1e9
    del x, dt, z, B, C, out, ws
    block_us = ssd_block_latency(torch, bm, I, dev, w, A, Dv, bias)
    return {
        "workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
        "d_state": w.d_state, "io_dtype": "bf16", "state_dtype": "f32",
        "ms_per_call": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "kernels_ms": {k: round(v, 4) for k, v in per.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(gbs_dom, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs_dom / HBM_PEAK_GBS, 4), "bytes_per_launch": io_bytes,
                     "traffic": profiled_traffic(profile=SSD_PROFILE, source=SSD_SOURCE,
                                                 key=f"hbm_bytes_per_dispatch_{dom}"),
                     "note": "the call's algorithmic bytes over the dominant kernel's time"},
        "hbm": {"algorithmic_bytes": io_bytes, "achieved_gbs": round(io_bytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(io_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": profiled_traffic(profile=SSD_PROFILE, source=SSD_SOURCE, key="hbm_bytes_per_call")},
        "mfma": {"flop_per_call": pages_flop, "achieved_tflops": round(pages_flop / (ms * 1e-3) / 1e12, 2),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(pages_flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                 "note": "the pages' count, 2 d_inner d_state per token and direction, over the whole call"},
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
        warm(g.replay, 3, torch)
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


def bench_ssd_conv(args, torch, bm, I, dev, stream):
    """Mamba-2 layers with untied directions and their short convolution, at the 1.3B layer's shape (120 heads
    of 32, state 128, the 4096-channel xBC stream, L = 65536): both layers fused (bimamba_ssd_conv_untied with
    the taps) against the two-pass pipeline (each layer's stream through bimamba_conv1d_bidir in its direction,
    then the same entry point without the convolution)."""
    L, H, P, N = 65536, 120, 32, 128
    xs = H * P + 2 * N
    sets = []
    for s_ in (61, 62):
        d = I.device_normals({"xbc": (1, L, xs), "dt": (1, L, H), "z": (1, L, H * P)}, seed=s_, io_dtype="bf16",
                             device=dev, scales={"dt": 0.5})
        A, Dv, bias = (torch.from_numpy(a).to(dev) for a in I.make_ssd_params(H, seed=s_ - 60))
        cw = torch.from_numpy(I.normal(s_, "conv_w", (xs, 4), 0.5, "f32")).to(dev)
        cb = torch.from_numpy(I.normal(s_, "conv_b", (xs,), 0.1, "f32")).to(dev)
        d.update(A=A, D=Dv, dt_bias=bias, cw=cw, cb=cb)
        sets.append(d)
    f, r = sets
    out_f, out_r = torch.empty(1, L, H * P, dtype=torch.bfloat16, device=dev), torch.empty(
        1, L, H * P, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(bm.bimamba_ssd_fwd_workspace_bytes(1, L, H, P, N), dtype=torch.uint8, device=dev)
    uf, ur = torch.empty_like(f["xbc"]), torch.empty_like(r["xbc"])

    def fused():
        bm.bimamba_ssd_conv_untied(f, r, out_f=out_f, out_r=out_r, workspace=ws, stream=stream)

    def conv_pass():
        bm.bimamba_conv1d_bidir(f["xbc"], f["cw"], f["cb"], None, None, out_f=uf, stream=stream)
        bm.bimamba_conv1d_bidir(r["xbc"], None, None, r["cw"], r["cb"], out_r=ur, stream=stream)

    def layers_unfused():
        bm.bimamba_ssd_conv_untied(dict(f, xbc=uf, cw=None, cb=None), dict(r, xbc=ur, cw=None, cb=None),
                                   out_f=out_f, out_r=out_r, workspace=ws, stream=stream)

    def timed(fn):
        warm(fn, 2, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_fused = timed(fused)
    ms_conv = timed(conv_pass)
    ms_layers = timed(layers_unfused)
    # algorithmic bytes of the fused call: per layer the stream read once, dt, z read once, out written once
    nbytes = 2 * L * (xs * 2 + H * 2 + 2 * H * P * 2)
    log(f"ssd conv layers (untied, fused): {ms_fused:.4f} ms; two-pass: conv {ms_conv:.4f} + layers "
        f"{ms_layers:.4f} ms")
    return {"workload": "ssd_conv_untied_long_64k_bf16", "seq_len": L, "nheads": H, "headdim": P, "d_state": N,
            "conv_channels": xs, "d_conv": 4, "layers": 2, "ms_per_call_fused": round(ms_fused, 4),
            "ms_two_pass": round(ms_conv + ms_layers, 4), "ms_conv_pass": round(ms_conv, 4),
            "ms_layers_unfused": round(ms_layers, 4),
            "tokens_per_s_fused": round(L / (ms_fused * 1e-3), 1),
            "hbm": {"algorithmic_bytes": nbytes, "achieved_gbs": round(nbytes / (ms_fused * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "traffic_fused": profiled_traffic(profile=SSDCONV_PROFILE, source=SSD_SOURCE,
                                                      key="hbm_bytes_per_call_fused"),
                    "traffic_two_pass": profiled_traffic(profile=SSDCONV_PROFILE, source=SSD_SOURCE,
                                                         key="hbm_bytes_per_call_two_pass")},
            "note": "two untied Mamba-2 layers (forward: causal conv, reverse: anti-causal conv, each its own "
                    "stream, dt, z and parameters); two-pass = the convolution kernel on each stream, then the "
                    "same layers reading the stored convolution output"}


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

    warm(step, args.warmup, torch)
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
    ap.add_argument("--cpu-channels", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ssd", action="store_true", help="skip the Mamba-2 (SSD) heads measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the batched and block-variant workloads reported beside the headline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--no-micro", action="store_true", help="skip the microbenchmarks")
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

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def timed_steps():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, ev0.elapsed_time(ev1) / args.steps

    # the same K steps after an idle second and only W warmup steps (the clock still climbing)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    time.sleep(1.0)
    for _ in range(args.warmup):
        step()
    ms_step_idle, _ = timed_steps()
    log(f"after an idle second and {args.warmup} warmup steps: {ms_step_idle:.4f} ms/step")

    nwarm = warm(step, args.warmup, torch)
    ms_step, ms_step_ev = timed_steps()
    log(f"warmup {nwarm} steps; timed {args.steps} steps: {ms_step:.4f} ms/step wall, {ms_step_ev:.4f} ms/step "
        f"events")
    # each call timed on its own (HIP events around it): the median and the minimum beside the mean
    evp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evp:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per_call = [e0.elapsed_time(e1) for e0, e1 in evp]
    log(f"per call: median {np.median(per_call):.4f} ms, min {min(per_call):.4f} ms")

    # the general-A path on the same inputs (reported beside the headline)
    warm(lambda: step(A_gen), 2, torch)
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

    warm(step_untied, 2, torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_untied()
    torch.cuda.synchronize()
    ms_step_untied = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"untied directions: {ms_step_untied:.4f} ms/step")

    # per-kernel attribution on the same stream: staged entry point, events between stages
    names = ("k_summary", "k_carry", "k_output")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    warm(step, args.warmup, torch)
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
    long_shape = w.name == "long_64k_bf16"
    traffic = profiled_traffic(elems) if long_shape else None
    gbs_out = abytes / t_out / 1e9
    roofline = {"bound": "hbm", "achieved": round(gbs_out, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs_out / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_output (output pass; the workload's A takes its geometric body)",
                "kernel_ms": round(per["k_output"], 4), "bytes_per_launch": abytes,
                "note": "the call's algorithmic bytes (each input read once, out written once) over the output "
                        "kernel's time"}
    micro = None if args.no_micro else bench_micro(torch, dev, stream)
    cnt = profiled_counters() if long_shape else None
    valu = None
    if cnt:
        ghz = micro["clock_ghz_under_fma_load"] if micro else NOMINAL_CLOCK_GHZ
        clk = per["k_output"] * 1e-3 * ghz * 1e9 / cnt["instructions_per_simd"]
        valu = {"kernel": "k_output", "lane_ops_per_element": cnt["lane_ops_per_element"],
                "instructions_per_simd": cnt["instructions_per_simd"], "clock_ghz": ghz,
                "clk_per_instruction": round(clk, 3)}
        if micro:
            floor = micro["fma_clk_per_instruction_4waves"]
            valu.update(issue_clk_per_instruction=floor, frac=round(floor / clk, 4))
        valu["note"] = ("wavefront VALU instructions of one launch per SIMD (committed SQ counters of this kernel "
                        "source) and the clocks each took at the shader clock measured under load (micro), against "
                        "independent VGPR-operand FMAs issued at 4 wavefronts per SIMD (micro); the kernel's "
                        "transcendentals issue at a quarter of that rate")
    hbm_gbs = abytes / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": nwarm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io_dtype if w.io_dtype != "f32" else "f32",
        "data": "synthetic (seeded N(0,1) activations, A[d,n]=-(n+1), D=1, log-uniform softplus(dt_bias))",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner,
                   "d_state": w.d_state, "io_dtype": w.io_dtype, "state_dtype": "f32"},
        "roofline": roofline,
        "valu": valu,
        "hbm": {"algorithmic_bytes": abytes, "achieved_gbs": round(hbm_gbs, 1),
                "frac_of_peak": round(hbm_gbs / HBM_PEAK_GBS, 4), "peak_gbs": HBM_PEAK_GBS,
                "traffic": profiled_traffic(elems, key="hbm_bytes_per_call") if long_shape else None},
        "kernels_ms": {k: round(v, 4) for k, v in per.items()},
        "general_A": {"ms_per_step": round(ms_step_gen, 4), "tokens_per_s": round(tokens / (ms_step_gen * 1e-3), 1),
                      "note": "A[d,n] = -(n+1)*(1+0.2*U(-1,1)): no per-channel geometric structure, one exp per "
                              "(token, channel, state) in each pass"},
        "ms_per_step_events": round(ms_step_ev, 4),
        "ms_per_step_after_idle": round(ms_step_idle, 4),
        "ms_per_call_median": round(float(np.median(per_call)), 4),
        "ms_per_call_min": round(float(min(per_call)), 4),
        "untied": {"ms_per_step": round(ms_step_untied, 4),
                   "tokens_per_s": round(tokens / (ms_step_untied * 1e-3), 1),
                   "note": "each direction its own x, dt, B, C, z, A, D, dt_bias and its own gated output "
                           "(bimamba_scan_fwd_untied): a forward-only and a reverse-only pass, twice the "
                           "activation bytes and no shared abar"},
    }
    if micro:
        line["micro"] = micro
    if not args.no_ssd:
        del x, dt, z, B, C, out, out_r, rev_set, fwd_set, ws
        torch.cuda.empty_cache()
        line["ssd"] = bench_ssd(args, torch, bm, I, dev, stream)
        torch.cuda.empty_cache()
        line["conv"] = bench_conv(args, torch, bm, I, dev, stream)
        torch.cuda.empty_cache()
        line["ssd_conv_layers"] = bench_ssd_conv(args, torch, bm, I, dev, stream)
    if not args.no_configs and w.name == "long_64k_bf16":
        torch.cuda.empty_cache()
        other = {"batched_8k_bf16": bench_batched(args, torch, bm, I, dev, stream)}
        torch.cuda.empty_cache()
        bl = bench_block(argparse.Namespace(steps=3, warmup=1), I.WORKLOADS["block_32k_bf16"], torch, bm, I, dev)
        other["block_32k_bf16"] = {k: bl[k] for k in ("value", "unit", "ms_per_step", "us_per_block_graph",
                                                       "us_per_block_eager", "us_per_block_call_graph")}
        other["block_32k_bf16"]["metric"] = bl["metric"]
        if micro:
            other["block_32k_bf16"]["empty_kernel_graph_us"] = micro["empty_kernel_graph_us"]
        line["other_configs"] = other
    if not args.no_cpu_baseline:
        nw = host_workers()
        log(f"cpu baseline: oracle on one thread ({args.cpu_channels} channels), then the whole workload on {nw} "
            f"processes")
        line["cpu_baseline"] = cpu_baseline(inp, w.seqlen, w.d_inner, min(args.cpu_channels, w.d_inner), nw)
        log(f"cpu baseline: {line['cpu_baseline']['sample']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
