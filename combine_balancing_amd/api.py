"""Tensor-level calls onto the mep C ABI.

Each function checks dtypes, devices and sizes of torch tensors, allocates
outputs when none are given, and calls the matching C entry point on the
current stream (or the stream passed). No arithmetic of the method happens
here. bf16 rows may be passed as torch.bfloat16 or as int16/uint16 bit
patterns.
"""
from __future__ import annotations

import torch

from . import _binding as B

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _stream_handle(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtypes, numel=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in (dtypes if isinstance(dtypes, tuple) else (dtypes,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _opt(t, name, dtypes, numel=None):
    return None if t is None else _need(t, name, dtypes, numel)


def plan_workspace(R, E, S, K, device=None):
    n = B.mep_plan_workspace_size(R, E, S, K)
    if n == 0:
        raise ValueError(f"unsupported plan sizes R={R} E={E} S={S} K={K}")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def plan_outputs(R, E, S, K, device=None, with_routes=True):
    dev = device or "cuda"
    C = S * K
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(
        expert_count=torch.empty(E, **i32), rank_load=torch.empty(R, **i32),
        inst_count=torch.empty(R, **i32), inst_expert=torch.empty(R, E, **i32),
        inst_cu=torch.empty(R, E + 1, **i32), inst_gid_base=torch.empty(R + 1, **i32),
        send_pos=torch.empty(C, **i32), send_count=torch.empty(R, **i32),
        recv_pos=torch.empty(C, **i32), recv_count=torch.empty(R, **i32))
    if with_routes:
        out["route_dest"] = torch.empty(R * C, **i32)
        out["route_slot"] = torch.empty(R * C, **i32)
    else:
        out["route_dest"] = out["route_slot"] = None
    return out


def plan(topk_ids, R, E, S, K, my_rank=0, workspace=None, out=None, stream=None,
         with_routes=True):
    """mep_plan on device int32 topk_ids [R*S*K]. Returns the output dict."""
    N = R * S * K
    ids = _need(topk_ids, "topk_ids", torch.int32, N)
    if workspace is None:
        workspace = plan_workspace(R, E, S, K, topk_ids.device)
    if out is None:
        out = plan_outputs(R, E, S, K, topk_ids.device, with_routes)
    C = S * K
    o = out
    rc = B.mep_plan(
        R, E, S, K, my_rank, ids, _need(workspace, "workspace", torch.uint8),
        workspace.numel(),
        _need(o["expert_count"], "expert_count", torch.int32, E),
        _need(o["rank_load"], "rank_load", torch.int32, R),
        _opt(o["route_dest"], "route_dest", torch.int32, N),
        _opt(o["route_slot"], "route_slot", torch.int32, N),
        _need(o["inst_count"], "inst_count", torch.int32, R),
        _need(o["inst_expert"], "inst_expert", torch.int32, R * E),
        _need(o["inst_cu"], "inst_cu", torch.int32, R * (E + 1)),
        _need(o["inst_gid_base"], "inst_gid_base", torch.int32, R + 1),
        _need(o["send_pos"], "send_pos", torch.int32, C),
        _need(o["send_count"], "send_count", torch.int32, R),
        _need(o["recv_pos"], "recv_pos", torch.int32, C),
        _need(o["recv_count"], "recv_count", torch.int32, R),
        _stream_handle(stream))
    B.check("mep_plan", rc)
    return out


def plan_noalloc(topk_ids, R, E, S, K, my_rank=0, out=None, stream=None, with_routes=True):
    """mep_plan_noalloc: mep_plan with its workspace in the library's static
    device array (no workspace argument, nothing allocated by the library).
    Outputs are allocated here only when `out` is not given."""
    N = R * S * K
    ids = _need(topk_ids, "topk_ids", torch.int32, N)
    if out is None:
        out = plan_outputs(R, E, S, K, topk_ids.device, with_routes)
    C = S * K
    o = out
    rc = B.mep_plan_noalloc(
        R, E, S, K, my_rank, ids,
        _need(o["expert_count"], "expert_count", torch.int32, E),
        _need(o["rank_load"], "rank_load", torch.int32, R),
        _opt(o["route_dest"], "route_dest", torch.int32, N),
        _opt(o["route_slot"], "route_slot", torch.int32, N),
        _need(o["inst_count"], "inst_count", torch.int32, R),
        _need(o["inst_expert"], "inst_expert", torch.int32, R * E),
        _need(o["inst_cu"], "inst_cu", torch.int32, R * (E + 1)),
        _need(o["inst_gid_base"], "inst_gid_base", torch.int32, R + 1),
        _need(o["send_pos"], "send_pos", torch.int32, C),
        _need(o["send_count"], "send_count", torch.int32, R),
        _need(o["recv_pos"], "recv_pos", torch.int32, C),
        _need(o["recv_count"], "recv_count", torch.int32, R),
        _stream_handle(stream))
    B.check("mep_plan_noalloc", rc)
    return out


_SCALE_CODES = {torch.float32: B.MEP_SCALE_F32, torch.bfloat16: B.MEP_SCALE_BF16,
                torch.float16: B.MEP_SCALE_F16}


def remap_prune(expert_ids, eplb_table, world_size, place_per_rank, local_rank_id,
                balance_mode, expert_scales=None, pruning_threshold=None,
                active_mask=None, scale_dtype=None, want_send=True, out=None,
                stream=None):
    """mep_remap_prune. expert_ids [BS,K] int32, eplb_table [E,F] int32.

    expert_scales: float32 / bfloat16 / float16 tensor [BS,K], or raw 16-bit
    patterns with scale_dtype given ("bf16" or "fp16").
    """
    BS, K = expert_ids.shape
    E, F = eplb_table.shape
    dev = expert_ids.device
    if expert_scales is not None:
        if scale_dtype is None:
            code = _SCALE_CODES[expert_scales.dtype]
        else:
            code = {"fp32": B.MEP_SCALE_F32, "bf16": B.MEP_SCALE_BF16,
                    "fp16": B.MEP_SCALE_F16}[scale_dtype]
        sc = _need(expert_scales, "expert_scales",
                   (torch.float32, torch.bfloat16, torch.float16, torch.int16, torch.uint16),
                   BS * K)
    else:
        code, sc = B.MEP_SCALE_BF16, None
    if out is None:
        out = dict(balanced_ids=torch.empty(BS, K, dtype=torch.int32, device=dev),
                   balanced_mask=torch.empty(BS, K, dtype=torch.uint8, device=dev))
        if want_send:
            out["send_pos"] = torch.empty(BS * K, dtype=torch.int32, device=dev)
            out["send_count"] = torch.empty(world_size, dtype=torch.int32, device=dev)
    rc = B.mep_remap_prune(
        BS, K, E, F, world_size, place_per_rank, local_rank_id, balance_mode,
        _need(expert_ids, "expert_ids", torch.int32), _need(eplb_table, "eplb_table", torch.int32),
        sc, code, _opt(pruning_threshold, "pruning_threshold", torch.float32, K),
        _opt(active_mask, "active_mask", (torch.uint8, torch.bool), BS),
        _need(out["balanced_ids"], "balanced_ids", torch.int32, BS * K),
        _need(out["balanced_mask"], "balanced_mask", (torch.uint8, torch.bool), BS * K),
        _opt(out.get("send_pos"), "send_pos", torch.int32, BS * K),
        _opt(out.get("send_count"), "send_count", torch.int32, world_size),
        _stream_handle(stream))
    B.check("mep_remap_prune", rc)
    return out


def dispatch(K, x=None, send_pos=None, send_buf=None, recv_raw=None, recv_pos=None,
             recv_grouped=None, stream=None):
    """mep_dispatch: pack (x -> send_buf) and/or group (recv_raw -> recv_grouped).

    Allocates send_buf [T*K,H] / recv_grouped [n,H] when not given (pack leaves
    rows not named by send_pos untouched, so a fresh buffer is zero-filled).
    Returns (send_buf, recv_grouped).
    """
    if x is None and recv_raw is None:
        raise ValueError("nothing to do: give x and/or recv_raw")
    T = H = 0
    if x is not None:
        T, H = x.shape
        if send_buf is None:
            send_buf = torch.zeros(T * K, H, dtype=x.dtype, device=x.device)
        # the send buffer holds every row send_pos names: T*K rows for the
        # plan's map, fewer for a dedup map
        if send_buf.dim() != 2 or send_buf.shape[1] != H:
            raise ValueError("send_buf must be [rows, H]")
    n = 0
    if recv_raw is not None:
        n_raw, H2 = recv_raw.shape
        if x is not None and H2 != H:
            raise ValueError("x and recv_raw disagree on H")
        H = H2
        # grouped rows: one per recv_pos entry (the arrival buffer may be
        # shorter when a dedup map fans rows out)
        n = recv_pos.numel() if recv_pos is not None else n_raw
        if recv_grouped is None:
            recv_grouped = torch.empty(n, H, dtype=recv_raw.dtype, device=recv_raw.device)
    # the library bounds the pack's stores by send_buf's rows and the
    # grouping's reads by recv_raw's rows
    n_send = send_buf.shape[0] if x is not None else 0
    n_raw = recv_raw.shape[0] if recv_raw is not None else 0
    rc = B.mep_dispatch(
        T, K, H, _opt(x, "x", _BF16_LIKE),
        _opt(send_pos, "send_pos", torch.int32, T * K if x is not None else None),
        _opt(send_buf, "send_buf", _BF16_LIKE), n_send,
        n, _opt(recv_pos, "recv_pos", torch.int32, n if recv_raw is not None else None),
        _opt(recv_raw, "recv_raw", _BF16_LIKE), n_raw,
        _opt(recv_grouped, "recv_grouped", _BF16_LIKE, n * H if recv_raw is not None else None),
        _stream_handle(stream))
    B.check("mep_dispatch", rc)
    return send_buf, recv_grouped


def combine(y_ret, send_pos, scores, out_bf16=True, out_f32=False, stream=None):
    """mep_combine. y_ret [n_y,H] bf16 rows, send_pos [T*K], scores [T,K] fp32.

    out_bf16/out_f32: True to allocate, a tensor to write into, or False/None.
    Returns (out_bf16, out_f32).
    """
    T, K = scores.shape
    n_y, H = y_ret.shape
    dev = y_ret.device
    if out_bf16 is True:
        out_bf16 = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    elif out_bf16 is False:
        out_bf16 = None
    if out_f32 is True:
        out_f32 = torch.empty(T, H, dtype=torch.float32, device=dev)
    elif out_f32 is False:
        out_f32 = None
    rc = B.mep_combine(
        T, K, H, _need(y_ret, "y_ret", _BF16_LIKE), n_y,
        _need(send_pos, "send_pos", torch.int32, T * K),
        _need(scores, "scores", torch.float32, T * K),
        _opt(out_bf16, "out_bf16", _BF16_LIKE, T * H),
        _opt(out_f32, "out_f32", torch.float32, T * H),
        _stream_handle(stream))
    B.check("mep_combine", rc)
    return out_bf16, out_f32


def peer_table(bufs):
    """Device array of row-buffer addresses (one per rank) for the zero-copy
    calls. `bufs`: a list of R device tensors, or one [R, C, H] tensor.
    The table holds raw addresses: the caller keeps the buffers alive for as
    long as the table is used."""
    if isinstance(bufs, torch.Tensor):
        bufs = list(bufs.unbind(0))
    for b in bufs:
        _need(b, "peer buffer", _BF16_LIKE)
    ptrs = torch.tensor([b.data_ptr() for b in bufs], dtype=torch.int64)
    return ptrs.to(bufs[0].device)


def dispatch_to_peers(K, x, route_dest, route_slot, peers, C, stream=None):
    """mep_dispatch_to_peers. x [T,H]; route_dest/route_slot [T*K] (this
    rank's routes); peers: device pointer table from peer_table()."""
    T, H = x.shape
    R = peers.numel()
    rc = B.mep_dispatch_to_peers(
        T, K, H, R, C, _need(x, "x", _BF16_LIKE),
        _need(route_dest, "route_dest", torch.int32, T * K),
        _need(route_slot, "route_slot", torch.int32, T * K),
        _need(peers, "peers", torch.int64, R), _stream_handle(stream))
    B.check("mep_dispatch_to_peers", rc)


def combine_from_peers(peers, C, H, route_dest, route_slot, scores, out_bf16=True, out_f32=False,
                       stream=None):
    """mep_combine_from_peers. Returns (out_bf16, out_f32)."""
    T, K = scores.shape
    R = peers.numel()
    dev = scores.device
    if out_bf16 is True:
        out_bf16 = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    elif out_bf16 is False:
        out_bf16 = None
    if out_f32 is True:
        out_f32 = torch.empty(T, H, dtype=torch.float32, device=dev)
    elif out_f32 is False:
        out_f32 = None
    rc = B.mep_combine_from_peers(
        T, K, H, R, C, _need(peers, "peers", torch.int64, R),
        _need(route_dest, "route_dest", torch.int32, T * K),
        _need(route_slot, "route_slot", torch.int32, T * K),
        _need(scores, "scores", torch.float32, T * K),
        _opt(out_bf16, "out_bf16", _BF16_LIKE, T * H), _opt(out_f32, "out_f32", torch.float32, T * H),
        _stream_handle(stream))
    B.check("mep_combine_from_peers", rc)
    return out_bf16, out_f32


def ungroup(y_grouped, recv_pos, y_arrival=None, stream=None):
    """mep_ungroup: y_arrival[recv_pos[t]] = y_grouped[t]."""
    n, H = y_grouped.shape
    if y_arrival is None:
        y_arrival = torch.empty_like(y_grouped)
    rc = B.mep_ungroup(n, H, _need(recv_pos, "recv_pos", torch.int32, n),
                       _need(y_grouped, "y_grouped", _BF16_LIKE),
                       _need(y_arrival, "y_arrival", _BF16_LIKE, n * H), _stream_handle(stream))
    B.check("mep_ungroup", rc)
    return y_arrival


def combine_add_rmsnorm(y_ret, send_pos, scores, residual, gamma, eps=1e-6, x_out=True,
                        y_out=None, rstd_out=True, stream=None):
    """mep_combine_add_rmsnorm. Returns (y_out, x_out, rstd_out); x_out and
    rstd_out are None when passed as False."""
    T, K = scores.shape
    n_y, H = (0, residual.shape[-1]) if y_ret is None else y_ret.shape
    dev = scores.device
    if y_out is None:
        y_out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    if x_out is True:
        x_out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    elif x_out is False:
        x_out = None
    if rstd_out is True:
        rstd_out = torch.empty(T, dtype=torch.float32, device=dev)
    elif rstd_out is False:
        rstd_out = None
    rc = B.mep_combine_add_rmsnorm(
        T, K, H, _opt(y_ret, "y_ret", _BF16_LIKE), n_y,
        _need(send_pos, "send_pos", torch.int32, T * K),
        _need(scores, "scores", torch.float32, T * K),
        _need(residual, "residual", _BF16_LIKE, T * H), _need(gamma, "gamma", _BF16_LIKE, H),
        float(eps), _opt(x_out, "x_out", _BF16_LIKE, T * H), _need(y_out, "y_out", _BF16_LIKE, T * H),
        _opt(rstd_out, "rstd_out", torch.float32, T), _stream_handle(stream))
    B.check("mep_combine_add_rmsnorm", rc)
    return y_out, x_out, rstd_out


def quant_msg_bytes(H):
    """Bytes of one int8 token message (Align512(Align32(H) + 4))."""
    return B.mep_quant_msg_bytes(H)


def dispatch_quant(K, x, send_pos, send_msgs=None, smooth=None, route_expert=None, n_rows=None,
                   stream=None):
    """mep_dispatch_quant. x [T,H] bf16; send_pos [T*K]; smooth [E,H] fp32
    and route_expert [T*K] (optional, together). Returns send_msgs
    [n_rows, msg_bytes] uint8 (allocated if not given)."""
    T, H = x.shape
    if send_msgs is None:
        n_rows = T * K if n_rows is None else n_rows
        send_msgs = torch.zeros(n_rows, quant_msg_bytes(H), dtype=torch.uint8, device=x.device)
    n_rows, msg_bytes = send_msgs.shape
    E = 0 if smooth is None else smooth.shape[0]
    rc = B.mep_dispatch_quant(
        T, K, H, _need(x, "x", _BF16_LIKE), _opt(smooth, "smooth", torch.float32),
        E, _opt(route_expert, "route_expert", torch.int32, T * K),
        _need(send_pos, "send_pos", torch.int32, T * K), n_rows, msg_bytes,
        _need(send_msgs, "send_msgs", torch.uint8), _stream_handle(stream))
    B.check("mep_dispatch_quant", rc)
    return send_msgs


def group_quant(recv_msgs, recv_pos, H, x_q=None, scales=None, stream=None):
    """mep_group_quant. recv_msgs [n_msgs, msg_bytes] uint8 in arrival order,
    recv_pos [n]. Returns (x_q [n, H] int8, scales [n] fp32)."""
    n_msgs, msg_bytes = recv_msgs.shape
    n = recv_pos.numel()
    dev = recv_msgs.device
    if x_q is None:
        x_q = torch.empty(n, H, dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty(n, dtype=torch.float32, device=dev)
    rc = B.mep_group_quant(n, H, msg_bytes, _need(recv_pos, "recv_pos", torch.int32, n), n_msgs,
                           _need(recv_msgs, "recv_msgs", torch.uint8),
                           _need(x_q, "x_q", (torch.int8, torch.uint8), n * H),
                           _need(scales, "scales", torch.float32, n), _stream_handle(stream))
    B.check("mep_group_quant", rc)
    return x_q, scales


def plan_weight_rows(plan_out, R, E, prefetch_slots, inst_wrow=None, stream=None):
    """mep_plan_weight_rows on mep_plan's outputs with B = prefetch_slots.
    Returns inst_wrow [R, E]."""
    ic, ie = plan_out["inst_count"], plan_out["inst_expert"]
    if inst_wrow is None:
        inst_wrow = torch.empty(R, E, dtype=torch.int32, device=ic.device)
    rc = B.mep_plan_weight_rows(R, E, prefetch_slots, _need(ic, "inst_count", torch.int32, R),
                                _need(ie, "inst_expert", torch.int32, R * E),
                                _need(inst_wrow, "inst_wrow", torch.int32, R * E),
                                _stream_handle(stream))
    B.check("mep_plan_weight_rows", rc)
    return inst_wrow


def plan_dedup(plan_out, R, S, K, my_rank, workspace=None, out=None, stream=None):
    """mep_plan_dedup on mep_plan's route maps. Returns dict(dpack_pos,
    dsend_count, drecv_pos, drecv_count)."""
    rd, rs = plan_out["route_dest"], plan_out["route_slot"]
    if rd is None or rs is None:
        raise ValueError("the plan must carry route_dest and route_slot")
    dev = rd.device
    C = S * K
    if workspace is None:
        n = B.mep_plan_dedup_workspace_size(R, S, K)
        if n == 0:
            raise ValueError(f"unsupported dedup sizes R={R} S={S} K={K}")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(dpack_pos=torch.empty(C, **i32), dsend_count=torch.empty(R, **i32),
                   drecv_pos=torch.empty(C, **i32), drecv_count=torch.empty(R, **i32))
    rc = B.mep_plan_dedup(
        R, S, K, my_rank, _need(rd, "route_dest", torch.int32, R * C),
        _need(rs, "route_slot", torch.int32, R * C), _need(workspace, "workspace", torch.uint8),
        workspace.numel(), _need(out["dpack_pos"], "dpack_pos", torch.int32, C),
        _need(out["dsend_count"], "dsend_count", torch.int32, R),
        _need(out["drecv_pos"], "drecv_pos", torch.int32, C),
        _need(out["drecv_count"], "drecv_count", torch.int32, R), _stream_handle(stream))
    B.check("mep_plan_dedup", rc)
    return out
