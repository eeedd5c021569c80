"""MoE expert layer for AMD Instinct MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP, C ABI declared in
``include/moe.h``); :mod:`.binding` is a thin ctypes layer over it that passes
torch device pointers and the current HIP stream.  Nothing here computes on
the host.
"""
from .binding import (MoEError, MoEShape, load_library, lib_path, workspace_size,  # noqa: F401
                      moe_route, moe_permute, moe_grouped_ffn_fwd, moe_combine,
                      moe_combine_bwd, moe_grouped_ffn_bwd, moe_permute_bwd, moe_route_bwd,
                      prof_enable, prof_select, prof_reset, prof_read, prof_names, OPS, DTYPES, GATES)
