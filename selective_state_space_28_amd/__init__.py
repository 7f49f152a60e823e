"""Selective state-space scan (S6) on MI355X: Python binding of libssm.

The functions carry the names of the C entry points in include/ssm.h and do
argument marshalling only (dtype/shape/device checks, output and workspace
allocation through torch, the current torch stream).  Every step of the
computation runs in the HIP kernels of libssm.so; if the library is missing
the calls raise instead of falling back to anything else.

    y, last = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias,
                           delta_softplus=True, h0=None, return_last_state=True)
    y = ssm_state_update(state, u, delta, A, B, C, D, z, delta_bias)
    y = ssm_conv_scan_fwd(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias)
    y = ssm_conv_state_update(conv_state, state, x, conv_w, conv_b, delta, A, B, C, D, z,
                              delta_bias)
    grads = ssm_scan_bwd(u, delta, A, B, C, D, z, delta_bias, dy=dy)
    y, last, ckpt = ssm_scan_fwd_ckpt(u, delta, A, B, C, D, z, delta_bias)
    grads = ssm_scan_bwd_ckpt(u, delta, A, B, C, D, z, delta_bias, ckpt=ckpt, dy=dy)
    y = ssm_ssd_scan_fwd(x, dt, A_head, B, C, D, z, dt_bias)
"""
from __future__ import annotations

from ._lib import SSM_BF16, SSM_F32, SsmError, header_functions, load, status_string  # noqa: F401
from .ops import (ssm_conv_scan_fwd, ssm_conv_state_update, ssm_scan_bwd,  # noqa: F401
                  ssm_scan_bwd_ckpt, ssm_scan_bwd_ckpt_workspace_bytes, ssm_scan_bwd_workspace_bytes,
                  ssm_scan_ckpt_bytes, ssm_scan_fwd, ssm_scan_fwd_ckpt, ssm_scan_fwd_noalloc,
                  ssm_scan_fwd_workspace_bytes,
                  ssm_ssd_scan_fwd, ssm_ssd_scan_fwd_workspace_bytes, ssm_state_update,
                  ssm_status_string)

__all__ = ["ssm_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_workspace_bytes", "ssm_state_update",
           "ssm_conv_scan_fwd", "ssm_conv_state_update", "ssm_scan_bwd",
           "ssm_scan_bwd_workspace_bytes", "ssm_scan_ckpt_bytes", "ssm_scan_fwd_ckpt",
           "ssm_scan_bwd_ckpt", "ssm_scan_bwd_ckpt_workspace_bytes", "ssm_ssd_scan_fwd", "ssm_ssd_scan_fwd_workspace_bytes",
           "ssm_status_string", "SsmError", "load"]
