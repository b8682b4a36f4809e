"""Selective-SSM scan for AMD MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (``include/ssm_scan.h``), with this
package as a thin torch binding: the forward scan, its backward with
recomputation from chunk-boundary states, and the single-token decode update
of the Mamba selective state-space model (Gu & Dao, arXiv 2312.00752).
"""
from ._lib import EXPORTS, LIB_PATH, SSMError, load  # noqa: F401
from .ops import (ConvScanFn, SelectiveScanFn, affine_scan, bidirectional_scan, chunk_len,  # noqa: F401
                  conv_selective_scan, scan_bwd, scan_bwd_conv, scan_fwd, scan_fwd_conv,
                  scan_fwd_plan, selective_scan, state_update)

__all__ = ["scan_fwd", "scan_bwd", "state_update", "selective_scan", "SelectiveScanFn",
           "bidirectional_scan", "scan_fwd_conv", "scan_bwd_conv", "conv_selective_scan",
           "ConvScanFn", "chunk_len", "scan_fwd_plan", "affine_scan", "load", "SSMError"]
