"""fp64 CPU oracle for the bidirectional selective scan (per-channel S6 and per-head Mamba-2).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the graft entry point's
smoke check and by the benchmark's CPU-baseline leg, never by the library.
"""
from .scan import (  # noqa: F401
    discretise,
    forward_scan,
    reverse_scan,
    scan_block,
    scan_fwd,
    scan_fwd_untied,
    silu,
    softplus,
)
from .conv import conv_anticausal, conv_bidir, conv_block, conv_causal  # noqa: F401
from .ssd import ssd_discretise, ssd_forward_scan, ssd_reverse_scan, ssd_scan_block, ssd_scan_fwd  # noqa: F401
