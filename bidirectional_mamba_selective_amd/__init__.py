"""MI355X-native bidirectional selective (S6) scan.

The compute lives in libbimamba.so (HIP kernels for gfx950, C ABI in
include/bimamba.h); this package holds its ctypes binding, the in-tree build
script and the seeded input generator used by the tests and the benchmark.
"""
from ._lib import (  # noqa: F401
    BIMAMBA_BF16,
    BIMAMBA_F32,
    FLAG_FWD_ONLY,
    FLAG_NO_SILU,
    FLAG_NO_GATE,
    FLAG_REV_ONLY,
    BimambaError,
    bimamba_conv1d_bidir,
    bimamba_conv1d_block,
    bimamba_scan_block,
    bimamba_scan_block_workspace_bytes,
    bimamba_scan_fwd,
    bimamba_scan_fwd_noalloc,
    bimamba_scan_fwd_stage,
    bimamba_scan_fwd_untied,
    bimamba_scan_fwd_workspace_bytes,
    bimamba_ssd_block,
    bimamba_ssd_block_workspace_bytes,
    bimamba_ssd_conv_untied,
    bimamba_ssd_fwd,
    bimamba_ssd_fwd_stage,
    bimamba_ssd_fwd_workspace_bytes,
    bimamba_status_string,
    bimamba_version,
    load,
)

__version__ = "0.1.0"
