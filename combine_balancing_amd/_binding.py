"""ctypes binding of libmep.so (include/mep.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmep.so")

MEP_OK, MEP_ERR_NULLPTR, MEP_ERR_PARAM, MEP_ERR_SHAPE, MEP_ERR_HIP = range(5)
MEP_SCALE_F32, MEP_SCALE_BF16, MEP_SCALE_F16 = 0, 1, 2
MEP_PLAN_NOALLOC_SCRATCH_BYTES = 4 << 20  # include/mep.h

_lib = None


class MepError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name} returned {code}: {msg}")
        self.code = code


def lib():
    """The loaded library. Raises if libmep.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m combine_balancing_amd.build` (hipcc, gfx950)")
    import torch  # noqa: F401  (load torch's HIP runtime first: one runtime per process)
    L = ctypes.CDLL(LIB_PATH)
    I, P, Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.mep_status_str.argtypes = [I]
    L.mep_status_str.restype = ctypes.c_char_p
    L.mep_version.argtypes = []
    L.mep_version.restype = I
    L.mep_plan_workspace_size.argtypes = [I, I, I, I]
    L.mep_plan_workspace_size.restype = Z
    L.mep_plan.argtypes = [I, I, I, I, I, P, P, Z] + [P] * 12 + [P]
    L.mep_plan.restype = I
    L.mep_plan_noalloc.argtypes = [I, I, I, I, I, P] + [P] * 12 + [P]
    L.mep_plan_noalloc.restype = I
    L.mep_remap_prune.argtypes = [I] * 8 + [P, P, P, I, P, P, P, P, P, P, P]
    L.mep_remap_prune.restype = I
    L.mep_dispatch.argtypes = [I, I, I, P, P, P, I, I, P, P, I, P, P]
    L.mep_dispatch.restype = I
    L.mep_combine.argtypes = [I, I, I, P, I, P, P, P, P, P]
    L.mep_combine.restype = I
    L.mep_dispatch_to_peers.argtypes = [I, I, I, I, I, P, P, P, P, P]
    L.mep_dispatch_to_peers.restype = I
    L.mep_combine_from_peers.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
    L.mep_combine_from_peers.restype = I
    L.mep_ungroup.argtypes = [I, I, P, P, P, P]
    L.mep_ungroup.restype = I
    L.mep_combine_add_rmsnorm.argtypes = [I, I, I, P, I, P, P, P, P, ctypes.c_float, P, P, P, P]
    L.mep_combine_add_rmsnorm.restype = I
    L.mep_quant_msg_bytes.argtypes = [I]
    L.mep_quant_msg_bytes.restype = Z
    L.mep_dispatch_quant.argtypes = [I, I, I, P, P, I, P, P, I, I, P, P]
    L.mep_dispatch_quant.restype = I
    L.mep_group_quant.argtypes = [I, I, I, P, I, P, P, P, P]
    L.mep_group_quant.restype = I
    L.mep_plan_weight_rows.argtypes = [I, I, I, P, P, P, P]
    L.mep_plan_weight_rows.restype = I
    L.mep_plan_dedup_workspace_size.argtypes = [I, I, I]
    L.mep_plan_dedup_workspace_size.restype = Z
    L.mep_plan_dedup.argtypes = [I, I, I, I, P, P, P, Z, P, P, P, P, P]
    L.mep_plan_dedup.restype = I
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().mep_status_str(code).decode()


def check(name: str, code: int) -> None:
    if code != MEP_OK:
        raise MepError(name, code, status_str(code))


# Raw entry points, same names and argument order as include/mep.h. Pointers
# are integers (device addresses) or None; stream is a hipStream_t integer.

def mep_plan_workspace_size(R, E, S, K) -> int:
    return lib().mep_plan_workspace_size(R, E, S, K)


def mep_plan(R, E, S, K, my_rank, topk_ids, workspace, workspace_bytes,
             expert_count, rank_load, route_dest, route_slot, inst_count,
             inst_expert, inst_cu, inst_gid_base, send_pos, send_count,
             recv_pos, recv_count, stream) -> int:
    return lib().mep_plan(R, E, S, K, my_rank, topk_ids, workspace, workspace_bytes,
                          expert_count, rank_load, route_dest, route_slot, inst_count,
                          inst_expert, inst_cu, inst_gid_base, send_pos, send_count,
                          recv_pos, recv_count, stream)


def mep_plan_noalloc(R, E, S, K, my_rank, topk_ids, expert_count, rank_load, route_dest,
                     route_slot, inst_count, inst_expert, inst_cu, inst_gid_base, send_pos,
                     send_count, recv_pos, recv_count, stream) -> int:
    return lib().mep_plan_noalloc(R, E, S, K, my_rank, topk_ids, expert_count, rank_load,
                                  route_dest, route_slot, inst_count, inst_expert, inst_cu,
                                  inst_gid_base, send_pos, send_count, recv_pos, recv_count,
                                  stream)


def mep_remap_prune(BS, K, E, F, world_size, place_per_rank, local_rank_id,
                    balance_mode, expert_ids, eplb_table, expert_scales, scale_dtype,
                    pruning_threshold, active_mask, balanced_ids, balanced_mask,
                    send_pos, send_count, stream) -> int:
    return lib().mep_remap_prune(BS, K, E, F, world_size, place_per_rank, local_rank_id,
                                 balance_mode, expert_ids, eplb_table, expert_scales,
                                 scale_dtype, pruning_threshold, active_mask, balanced_ids,
                                 balanced_mask, send_pos, send_count, stream)


def mep_dispatch(T, K, H, x, send_pos, send_buf, n_send, n_recv, recv_pos, recv_raw, n_raw,
                 recv_grouped, stream) -> int:
    return lib().mep_dispatch(T, K, H, x, send_pos, send_buf, n_send, n_recv, recv_pos,
                              recv_raw, n_raw, recv_grouped, stream)


def mep_combine(T, K, H, y_ret, n_y, send_pos, scores, out_bf16, out_f32, stream) -> int:
    return lib().mep_combine(T, K, H, y_ret, n_y, send_pos, scores, out_bf16, out_f32, stream)


def mep_dispatch_to_peers(T, K, H, R, C, x, route_dest, route_slot, peer_bufs, stream) -> int:
    return lib().mep_dispatch_to_peers(T, K, H, R, C, x, route_dest, route_slot, peer_bufs,
                                       stream)


def mep_combine_from_peers(T, K, H, R, C, peer_bufs, route_dest, route_slot, scores, out_bf16,
                           out_f32, stream) -> int:
    return lib().mep_combine_from_peers(T, K, H, R, C, peer_bufs, route_dest, route_slot, scores,
                                        out_bf16, out_f32, stream)


def mep_ungroup(n, H, recv_pos, y_grouped, y_arrival, stream) -> int:
    return lib().mep_ungroup(n, H, recv_pos, y_grouped, y_arrival, stream)


def mep_combine_add_rmsnorm(T, K, H, y_ret, n_y, send_pos, scores, residual, gamma, eps, x_out,
                            y_out, rstd_out, stream) -> int:
    return lib().mep_combine_add_rmsnorm(T, K, H, y_ret, n_y, send_pos, scores, residual, gamma,
                                         eps, x_out, y_out, rstd_out, stream)


def mep_quant_msg_bytes(H) -> int:
    return lib().mep_quant_msg_bytes(H)


def mep_dispatch_quant(T, K, H, x, smooth, E, route_expert, send_pos, n_rows, msg_bytes,
                       send_msgs, stream) -> int:
    return lib().mep_dispatch_quant(T, K, H, x, smooth, E, route_expert, send_pos, n_rows,
                                    msg_bytes, send_msgs, stream)


def mep_group_quant(n, H, msg_bytes, recv_pos, n_msgs, recv_msgs, x_q, scales, stream) -> int:
    return lib().mep_group_quant(n, H, msg_bytes, recv_pos, n_msgs, recv_msgs, x_q, scales,
                                 stream)


def mep_plan_weight_rows(R, E, B, inst_count, inst_expert, inst_wrow, stream) -> int:
    return lib().mep_plan_weight_rows(R, E, B, inst_count, inst_expert, inst_wrow, stream)


def mep_plan_dedup_workspace_size(R, S, K) -> int:
    return lib().mep_plan_dedup_workspace_size(R, S, K)


def mep_plan_dedup(R, S, K, my_rank, route_dest, route_slot, workspace, workspace_bytes,
                   dpack_pos, dsend_count, drecv_pos, drecv_count, stream) -> int:
    return lib().mep_plan_dedup(R, S, K, my_rank, route_dest, route_slot, workspace,
                                workspace_bytes, dpack_pos, dsend_count, drecv_pos, drecv_count,
                                stream)
