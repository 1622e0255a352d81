"""Host-side checks of bench.py's measurement bookkeeping (no GPU).

The roofline's algorithmic bytes, and the committed rocprofv3 summaries the bench reads its traffic and
instruction counts from: each summary must have been taken on the kernel source as it stands (its
recorded sha256 prefix), otherwise the bench reports those fields as null.
"""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes(bench):
    """Each input read once and out written once: x, dt, z, out (d_inner values each) and B, C (d_state
    each) per token in the I/O dtype, plus A [d_inner, d_state] and D, dt_bias [d_inner] in fp32."""
    per_token = 4 * 4096 * 2 + 2 * 16 * 2
    assert per_token == 32832
    assert bench.algorithmic_bytes(1, 65536, 4096, 16, 2) == 65536 * per_token + 4096 * 16 * 4 + 2 * 4096 * 4
    assert bench.algorithmic_bytes(1, 65536, 4096, 16, 2) == 2151972864
    assert bench.algorithmic_bytes(8, 8192, 2048, 16, 2) == 8 * 8192 * (4 * 2048 * 2 + 64) + 2048 * 16 * 4 + 2 * 2048 * 4


@pytest.mark.parametrize("profile, source, key", [
    ("k_output_long_64k_bf16_traffic.txt", "scan_kernels.hip", "hbm_bytes_per_dispatch"),
    ("k_output_long_64k_bf16_traffic.txt", "scan_kernels.hip", "hbm_bytes_per_call"),
    ("k_ssd_long_64k_bf16_traffic.txt", "ssd_kernels.hip", "hbm_bytes_per_dispatch_k_ssd_rsweep"),
    ("k_ssd_long_64k_bf16_traffic.txt", "ssd_kernels.hip", "hbm_bytes_per_call"),
    ("k_conv_long_64k_bf16_traffic.txt", "conv_kernels.hip", "hbm_bytes_per_dispatch"),
    ("k_ssd1_conv_long_64k_bf16_traffic.txt", "ssd_kernels.hip", "hbm_bytes_per_call_fused"),
    ("k_ssd1_conv_long_64k_bf16_traffic.txt", "ssd_kernels.hip", "hbm_bytes_per_call_two_pass"),
])
def test_traffic_summaries_match_the_kernel_sources(bench, profile, source, key):
    v = bench.profiled_traffic(profile=os.path.join(ROOT, "profiles", profile),
                               source=os.path.join(ROOT, "bidirectional_mamba_selective_amd", "csrc", source), key=key)
    assert v is not None, f"{profile}: {key} missing, or the summary was taken on another {source}"
    assert 1e8 < v < 1e11


def test_counter_summary_matches_the_kernel_source(bench):
    c = bench.profiled_counters()
    assert c is not None, "the output kernel's SQ counter summary is missing or stale"
    # lane operations per (token, channel, state): the state step alone is 6
    assert 6.0 < c["lane_ops_per_element"] < 12.0
    # instructions per SIMD = lane operations x elements / 64 lanes / 1024 SIMDs
    elems = 65536 * 4096 * 16
    assert abs(c["instructions_per_simd"] - c["lane_ops_per_element"] * elems / 64 / 1024) < 0.01 * c[
        "instructions_per_simd"]
