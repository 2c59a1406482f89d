"""MI355X-native routed-expert decode path over fp4 (e2m1) weights with E4M3 group scales,
and the dense FP8 projections of a decode layer.

The compute lives in ``libxp.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, ``include/xp.h``); :mod:`fp4_routed_expert_xp_amd.xp` binds it.
"""
from . import xp  # noqa: F401
from .xp import (  # noqa: F401
    XPError, dims, xp_combine, xp_down_combine, xp_down_rows, xp_gateup_rows, xp_gateup_rows_split,
    xp_get_tiers, xp_pack_matrix, xp_prefill_down, xp_prefill_gateup, xp_route_bucket, xp_route_gateup, xp_set_tiers, xp_status_string,
    xp_workspace_bytes, xp_workspace_layout, xp_fp8_pack, xp_fp8_packed_bytes, xp_fp8_rows,
    xp_gateup_rows_act16, xp_down_rows_act16, xp_combine_y16, xp_fp8_rows_f32,
)
