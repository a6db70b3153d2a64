"""libflare: FLARE / FLARE++ low-rank attention routing forward on MI355X.

The compute path is the C-ABI shared library ``libflare.so`` (hand-written
gfx950 HIP kernels); this package holds its sources (``csrc/``), its build
script and the Python binding with the same entry-point names.
"""
from .flare import (FLARE_BF16, FLARE_F32, FLARE_LAYOUT_BHND, FLARE_LAYOUT_BNHD, FLARE_OP_BACKWARD, FLARE_OP_DECODE,
                    FLARE_OP_ENCODE, FLARE_OP_FORWARD, FLARE_OP_PP_BACKWARD, FLARE_OP_PP_FORWARD, FLARE_OP_PP_QUERIES,
                    FLARE_PROBE_EXP, FLARE_PROBE_MFMA_BF16, FlareError, flare_attend, flare_backward,
                    flare_backward_ex, flare_copy_kernel, flare_decode, flare_decode_ex, flare_describe_plan,
                    flare_encode, flare_encode_ex, flare_forward, flare_forward_ex, flare_forward_noalloc,
                    flare_pp_backward, flare_pp_backward_ex, flare_pp_forward, flare_pp_forward_ex, flare_pp_queries,
                    flare_probe_lanes, flare_probe_peak, flare_read_kernel, flare_set_tuning, flare_timing_enable, flare_timing_read,
                    flare_workspace_size, lib, workspace_for)

__all__ = ["FLARE_BF16", "FLARE_F32", "FLARE_LAYOUT_BHND", "FLARE_LAYOUT_BNHD", "FLARE_OP_BACKWARD",
           "FLARE_OP_DECODE", "FLARE_OP_ENCODE", "FLARE_OP_FORWARD", "FLARE_OP_PP_BACKWARD", "FLARE_OP_PP_FORWARD",
           "FLARE_OP_PP_QUERIES", "FLARE_PROBE_EXP", "FLARE_PROBE_MFMA_BF16", "FlareError", "flare_attend",
           "flare_backward", "flare_backward_ex", "flare_copy_kernel", "flare_decode", "flare_decode_ex",
           "flare_describe_plan", "flare_encode", "flare_encode_ex", "flare_forward", "flare_forward_ex",
           "flare_forward_noalloc", "flare_pp_backward", "flare_pp_backward_ex", "flare_pp_forward",
           "flare_pp_forward_ex", "flare_pp_queries", "flare_probe_lanes", "flare_probe_peak", "flare_read_kernel",
           "flare_set_tuning",
           "flare_timing_enable", "flare_timing_read", "flare_workspace_size", "lib", "workspace_for"]
