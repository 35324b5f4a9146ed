"""MI355X-native Variational Linear Attention (VLA) recurrence: forward, decode
step and gradients.

The compute lives in ``libvla.so`` (hand-written gfx950 HIP kernels behind the
C ABI in ``include/vla.h``); this package is its thin Python binding.
"""
from ._binding import (NOALLOC_SCRATCH_BYTES, VLA_BF16, VLA_ERR_HIP, VLA_ERR_INVALID_ARG,
                       VLA_ERR_UNSUPPORTED, VLA_F32, VLA_OK, LIB_PATH, VLAError,
                       backward_workspace_size, baseline_workspace_size, load,
                       scan_workspace_size, vla_backward, vla_baseline,
                       vla_forward, vla_forward_memory, vla_forward_noalloc, vla_forward_penalty,
                       vla_forward_scan, vla_status_string, vla_step, workspace_size)
from .autograd import vla_attention

__all__ = ["vla_baseline", "baseline_workspace_size", "vla_forward", "vla_forward_penalty", "vla_forward_memory", "vla_forward_noalloc",
           "NOALLOC_SCRATCH_BYTES", "vla_step",
           "vla_backward", "vla_attention", "vla_forward_scan", "workspace_size",
           "backward_workspace_size", "scan_workspace_size", "vla_status_string", "VLAError", "load", "LIB_PATH",
           "VLA_OK", "VLA_ERR_INVALID_ARG", "VLA_ERR_UNSUPPORTED", "VLA_ERR_HIP",
           "VLA_F32", "VLA_BF16"]
