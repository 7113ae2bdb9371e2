"""Selective-scan forward (Mamba ``selective_scan_fn``) and its causal conv
prologue for AMD MI355X (gfx950): a C-ABI HIP library (``libssmscan.so``,
include/ssmscan.h) and a thin torch binding.

The operator follows the PaddleNLP Kernel operator-library guide, section 4.1
(selective_scan) and section 4.2 (causal_conv1d).
"""
from ._lib import SsmError, EXPORTS  # noqa: F401
from .binding import (  # noqa: F401
    causal_conv1d_fn,
    causal_conv1d_fwd,
    conv1d_selective_scan_fn,
    selective_scan_fn,
    ssm_scan_fwd,
    ssm_scan_fwd_complex,
)
