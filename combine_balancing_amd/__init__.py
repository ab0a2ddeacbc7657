"""Balanced expert-parallel MoE hot path on MI355X (gfx950).

The work is done by libmep.so (C ABI in include/mep.h, HIP kernels under
csrc/). This package is its binding: ``_binding`` holds the raw entry points
under their C names, ``api`` the tensor-level calls. Importing the package
does not load the library; the first call does, and raises if it has not
been built (``python -m combine_balancing_amd.build``).
"""
from .api import (combine, combine_add_rmsnorm, combine_from_peers, dispatch,  # noqa: F401
                  dispatch_quant, dispatch_to_peers, group_quant, peer_table, plan, plan_noalloc,
                  plan_outputs,
                  plan_dedup, plan_weight_rows, plan_workspace, quant_msg_bytes, remap_prune, ungroup)
from ._binding import MepError, lib  # noqa: F401
