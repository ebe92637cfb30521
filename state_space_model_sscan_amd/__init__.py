"""libsscan: the selective state-space scan (Mamba-1 and Mamba-2 SSD) for AMD MI355X.

The compute path is the HIP library libsscan.so (C ABI in include/sscan.h);
`binding` is its thin ctypes wrapper. `inputs` draws seeded synthetic inputs.
"""
from .binding import (BF16, F32, ConvDesc, Mamba1Desc, SSDDesc, SscanError, lib,  # noqa: F401
                      set_pointer_checks, sscan_conv1d_silu, sscan_gated_rmsnorm, sscan_mamba1_fwd,
                      sscan_mamba1_workspace_size, sscan_ssd_fwd, sscan_ssd_step, sscan_ssd_workspace_size,
                      sscan_step, ssd_state_key_first)
