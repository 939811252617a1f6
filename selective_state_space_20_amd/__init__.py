"""MI355X-native (gfx950) selective scan.

The computation lives in libsss.so (hand-written HIP kernels behind the C ABI of
include/sss.h); this package is its thin Python binding:

  * ``selective_scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None)`` -> (y, h_last);
    keywords ``delta_bias``, ``delta_softplus``, ``exact_zoh`` and ``layout="bdl"``
    (channel-major operands) select the options of ``selective_scan_fwd_ex``
  * ``selective_scan_bwd(x, delta, A, B, C, D, z, h0, dy=..., dh_last=None)`` -> gradients;
    ``states=`` on both calls keeps the forward's segment entering states for the gradients
    (``selective_scan_states_size`` bytes: selective_scan_fwd_save / selective_scan_bwd_saved)
  * ``selective_state_update(x, delta, A, B, C, D=None, z=None, state=...)`` -> y (one
    decode step; ``state`` is updated in place)
  * ``causal_conv1d_fwd(x, weight, bias=None, silu=False)`` -> out (the conv front end)
  * ``elementwise_scan(x, A, B, C, h0=None)`` -> (y, h_last)
  * ``*_workspace_size``, raw-pointer variants ``*_raw`` and ``status_string``.

``inputs`` holds the seeded synthetic workload generators.
"""
from ._lib import (EXPORTED, LIB_PATH, SSSError, SSS_BF16, SSS_DELTA_SOFTPLUS, SSS_EXACT_ZOH, SSS_F32, SSS_LAYOUT_BDL,
                   causal_conv1d_fwd, causal_conv1d_fwd_raw, elementwise_scan, elementwise_scan_raw,
                   selective_scan_bwd, selective_scan_bwd_raw, selective_scan_bwd_ex_raw, selective_scan_bwd_workspace_size,
                   selective_scan_fwd_ex_raw, selective_scan_fwd_noalloc_raw, selective_scan_states_size,
                   selective_scan_fwd_save_raw, selective_scan_bwd_saved_raw,
                   elementwise_scan_workspace_size, load, selective_scan_fwd, selective_scan_fwd_raw,
                   selective_scan_fwd_workspace_size, selective_scan_fwd_ex_workspace_size,
                   selective_state_update, selective_state_update_raw,
                   status_string)

__all__ = ["selective_scan_fwd", "selective_scan_bwd", "selective_scan_bwd_raw", "selective_scan_bwd_ex_raw", "selective_scan_bwd_workspace_size",
           "selective_state_update", "causal_conv1d_fwd", "causal_conv1d_fwd_raw", "selective_state_update_raw", "elementwise_scan",
           "selective_scan_fwd_workspace_size",
           "elementwise_scan_workspace_size", "selective_scan_fwd_raw", "elementwise_scan_raw", "status_string",
           "SSSError", "SSS_F32", "SSS_BF16", "SSS_EXACT_ZOH", "SSS_DELTA_SOFTPLUS", "SSS_LAYOUT_BDL",
           "selective_scan_fwd_ex_workspace_size", "selective_scan_fwd_ex_raw", "selective_scan_fwd_noalloc_raw",
           "selective_scan_states_size", "selective_scan_fwd_save_raw", "selective_scan_bwd_saved_raw",
           "LIB_PATH", "EXPORTED", "load"]
