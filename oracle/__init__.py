"""CPU oracle for the balanced expert-parallel MoE hot path.

TEST INFRASTRUCTURE ONLY: the slow, single-threaded C definition
(``oracle.c``) that the GPU library is checked against, with thin numpy
wrappers. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the GPU
library and never imports it.

Every function here checks shapes, allocates its outputs as numpy arrays and
calls the matching C function. Arithmetic lives in ``oracle.c`` only.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MEP_ORACLE_LIB names another build of oracle.c to load (the mutation
# check in tests/oracle_mutations.py loads oracle builds with planted
# mistakes this way, leaving the in-tree library alone)
LIB_PATH = os.environ.get("MEP_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no FMA contraction)."""
    import subprocess
    src = os.path.join(_HERE, "oracle.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_plan.argtypes = [I, I, I, I, I, P] + [P] * 12
    lib.oracle_plan.restype = I
    lib.oracle_remap_prune.argtypes = [I] * 8 + [P, P, P, I, P, P, P, P, P, P]
    lib.oracle_remap_prune.restype = I
    lib.oracle_pack.argtypes = [I, I, I, P, P, P]
    lib.oracle_pack.restype = I
    lib.oracle_group.argtypes = [I, I, P, P, P]
    lib.oracle_group.restype = I
    lib.oracle_combine.argtypes = [I, I, I, P, P, P, P, P]
    lib.oracle_combine.restype = I
    lib.oracle_push.argtypes = [I, I, I, I, I, P, P, P, P]
    lib.oracle_push.restype = I
    lib.oracle_pull_combine.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
    lib.oracle_pull_combine.restype = I
    lib.oracle_ungroup.argtypes = [I, I, P, P, P]
    lib.oracle_ungroup.restype = I
    lib.oracle_combine_add_rmsnorm.argtypes = [I, I, I, P, I, P, P, P, P, ctypes.c_double,
                                               P, P, P, P]
    lib.oracle_combine_add_rmsnorm.restype = I
    lib.oracle_dispatch_quant.argtypes = [I, I, I, P, P, I, P, P, I, I, P]
    lib.oracle_dispatch_quant.restype = I
    lib.oracle_group_quant.argtypes = [I, I, I, P, I, P, P, P]
    lib.oracle_group_quant.restype = I
    lib.oracle_weight_rows.argtypes = [I, I, I, P, P, P]
    lib.oracle_weight_rows.restype = I
    lib.oracle_plan_dedup.argtypes = [I, I, I, I, P, P, P, P, P, P]
    lib.oracle_plan_dedup.restype = I
    lib.oracle_bf16_from_float.argtypes = [P, P, ctypes.c_int64]
    lib.oracle_bf16_from_float.restype = None
    lib.oracle_float_from_fp16.argtypes = [P, P, ctypes.c_int64]
    lib.oracle_float_from_fp16.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def plan(topk_ids, R, E, S, K, m=0):
    """Global plan + rank m's send/receive maps (see oracle_plan in oracle.c).

    Returns a dict of int32 arrays: expert_count[E], rank_load[R],
    route_dest[N], route_slot[N], inst_count[R], inst_expert[R,E],
    inst_cu[R,E+1], inst_gid_base[R+1], send_pos[C], send_count[R],
    recv_pos[C], recv_count[R].
    """
    lib = _load()
    ids = _c(topk_ids, np.int32).reshape(-1)
    C = S * K
    N = R * C
    if ids.size != N:
        raise ValueError("topk_ids must hold R*S*K entries")
    out = dict(
        expert_count=np.zeros(E, np.int32), rank_load=np.zeros(R, np.int32),
        route_dest=np.zeros(N, np.int32), route_slot=np.zeros(N, np.int32),
        inst_count=np.zeros(R, np.int32), inst_expert=np.zeros((R, E), np.int32),
        inst_cu=np.zeros((R, E + 1), np.int32),
        inst_gid_base=np.zeros(R + 1, np.int32),
        send_pos=np.zeros(C, np.int32), send_count=np.zeros(R, np.int32),
        recv_pos=np.zeros(C, np.int32), recv_count=np.zeros(R, np.int32))
    keys = ["expert_count", "rank_load", "route_dest", "route_slot", "inst_count",
            "inst_expert", "inst_cu", "inst_gid_base", "send_pos", "send_count",
            "recv_pos", "recv_count"]
    rc = lib.oracle_plan(R, E, S, K, m, _p(ids), *[_p(out[k]) for k in keys])
    _check(rc, "oracle_plan")
    return out


SCALE_DTYPES = {"fp32": 0, "bf16": 1, "fp16": 2}


def remap_prune(expert_ids, eplb_table, world_size, place_per_rank,
                local_rank_id, balance_mode, expert_scales=None,
                scale_dtype="bf16", pruning_threshold=None, active_mask=None,
                want_send=True):
    """EPLB remap + prune + send map (see oracle_remap_prune in oracle.c).

    expert_scales: uint16 bit patterns for bf16/fp16, float32 for fp32.
    """
    lib = _load()
    ids = _c(expert_ids, np.int32)
    BS, K = ids.shape
    table = _c(eplb_table, np.int32)
    E, F = table.shape
    sdt = SCALE_DTYPES[scale_dtype]
    sc = None
    if expert_scales is not None:
        sc = _c(expert_scales, np.float32 if sdt == 0 else np.uint16)
        if sc.shape != (BS, K):
            raise ValueError("expert_scales must be [BS,K]")
    thr = None if pruning_threshold is None else _c(pruning_threshold, np.float32).reshape(-1)
    act = None if active_mask is None else _c(active_mask, np.uint8).reshape(-1)
    bal = np.zeros((BS, K), np.int32)
    mask = np.zeros((BS, K), np.uint8)
    sp = np.zeros(BS * K, np.int32) if want_send else None
    scnt = np.zeros(world_size, np.int32) if want_send else None
    rc = lib.oracle_remap_prune(BS, K, E, F, world_size, place_per_rank,
                                local_rank_id, balance_mode, _p(ids), _p(table),
                                _p(sc), sdt, _p(thr), _p(act), _p(bal), _p(mask),
                                _p(sp), _p(scnt))
    _check(rc, "oracle_remap_prune")
    out = dict(balanced_ids=bal, balanced_mask=mask)
    if want_send:
        out["send_pos"] = sp
        out["send_count"] = scnt
    return out


def pack(x, send_pos, K, n_rows=None):
    """send_buf[send_pos[t*K+k]] = x[t] (rows with send_pos < 0 skipped)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    sp = _c(send_pos, np.int32).reshape(-1)
    if sp.size != T * K:
        raise ValueError("send_pos must hold T*K entries")
    if n_rows is None:
        n_rows = T * K
    buf = np.zeros((n_rows, H), np.uint16)
    if sp.size and sp.max() >= n_rows:
        raise ValueError("send_pos beyond send buffer")
    _check(lib.oracle_pack(T, K, H, _p(x), _p(sp), _p(buf)), "oracle_pack")
    return buf


def group(recv_raw, recv_pos):
    """recv_grouped[t] = recv_raw[recv_pos[t]]."""
    lib = _load()
    raw = _c(recv_raw, np.uint16)
    rp = _c(recv_pos, np.int32).reshape(-1)
    H = raw.shape[1]
    if rp.size and (rp.min() < 0 or rp.max() >= raw.shape[0]):
        raise ValueError("recv_pos out of range")
    out = np.zeros((rp.size, H), np.uint16)
    _check(lib.oracle_group(rp.size, H, _p(rp), _p(raw), _p(out)), "oracle_group")
    return out


def combine(y_ret, send_pos, scores, want_bf16=True, want_f32=True):
    """Score-weighted K-way reduction (see oracle_combine in oracle.c)."""
    lib = _load()
    y = _c(y_ret, np.uint16)
    sc = _c(scores, np.float32)
    T, K = sc.shape
    H = y.shape[1]
    sp = _c(send_pos, np.int32).reshape(-1)
    if sp.size != T * K:
        raise ValueError("send_pos must hold T*K entries")
    if sp.size and sp.max() >= y.shape[0]:
        raise ValueError("send_pos beyond y_ret")
    ob = np.zeros((T, H), np.uint16) if want_bf16 else None
    of = np.zeros((T, H), np.float32) if want_f32 else None
    _check(lib.oracle_combine(T, K, H, _p(y), _p(sp), _p(sc), _p(ob), _p(of)),
           "oracle_combine")
    return ob, of


def push(x, route_dest, route_slot, K, R, C, grouped=None):
    """Zero-copy dispatch into all R grouped buffers [R, C, H] (oracle_push)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    rd = _c(route_dest, np.int32).reshape(-1)
    rs = _c(route_slot, np.int32).reshape(-1)
    if rd.size != T * K or rs.size != T * K:
        raise ValueError("route maps must hold T*K entries")
    if grouped is None:
        grouped = np.zeros((R, C, H), np.uint16)
    _check(lib.oracle_push(T, K, H, R, C, _p(x), _p(rd), _p(rs), _p(grouped)), "oracle_push")
    return grouped


def pull_combine(grouped, route_dest, route_slot, scores, want_bf16=True, want_f32=True):
    """Zero-copy combine from grouped buffers [R, C, H] (oracle_pull_combine)."""
    lib = _load()
    g = _c(grouped, np.uint16)
    R, C, H = g.shape
    sc = _c(scores, np.float32)
    T, K = sc.shape
    rd = _c(route_dest, np.int32).reshape(-1)
    rs = _c(route_slot, np.int32).reshape(-1)
    ob = np.zeros((T, H), np.uint16) if want_bf16 else None
    of = np.zeros((T, H), np.float32) if want_f32 else None
    _check(lib.oracle_pull_combine(T, K, H, R, C, _p(g), _p(rd), _p(rs), _p(sc), _p(ob), _p(of)),
           "oracle_pull_combine")
    return ob, of


def ungroup(y_grouped, recv_pos):
    """y_arrival[recv_pos[t]] = y_grouped[t] (oracle_ungroup)."""
    lib = _load()
    y = _c(y_grouped, np.uint16)
    rp = _c(recv_pos, np.int32).reshape(-1)
    out = np.zeros_like(y)
    _check(lib.oracle_ungroup(rp.size, y.shape[1], _p(rp), _p(y), _p(out)), "oracle_ungroup")
    return out


def combine_add_rmsnorm(y_ret, send_pos, scores, residual, gamma, eps, n_y=None):
    """Combine + residual add + RMSNorm (oracle_combine_add_rmsnorm).
    Returns dict(x_out bf16 [T,H], x_f32 [T,H], rstd float64 [T], y float64 [T,H])."""
    lib = _load()
    y = _c(y_ret, np.uint16)
    sc = _c(scores, np.float32)
    T, K = sc.shape
    H = y.shape[1]
    sp = _c(send_pos, np.int32).reshape(-1)
    res = _c(residual, np.uint16).reshape(T, H)
    g = _c(gamma, np.uint16).reshape(H)
    if sp.size != T * K:
        raise ValueError("send_pos must hold T*K entries")
    n_y = y.shape[0] if n_y is None else n_y
    out = {"x_out": np.zeros((T, H), np.uint16), "x_f32": np.zeros((T, H), np.float32),
           "rstd": np.zeros(T, np.float64), "y": np.zeros((T, H), np.float64)}
    _check(lib.oracle_combine_add_rmsnorm(T, K, H, _p(y), n_y, _p(sp), _p(sc), _p(res), _p(g),
                                          float(eps), _p(out["x_out"]), _p(out["x_f32"]),
                                          _p(out["rstd"]), _p(out["y"])),
           "oracle_combine_add_rmsnorm")
    return out


def quant_msg_bytes(H):
    """Message row size of the int8 dispatch: Align512(Align32(H) + 4)."""
    return ((H + 31) // 32 * 32 + 4 + 511) // 512 * 512


def dispatch_quant(x, send_pos, K, smooth=None, route_expert=None, n_rows=None, msg_bytes=None,
                   msgs=None):
    """int8 pack (oracle_dispatch_quant). Returns the message rows
    [n_rows, msg_bytes] uint8 (bytes the oracle does not write stay as given,
    zero for a fresh buffer)."""
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    sp = _c(send_pos, np.int32).reshape(-1)
    if sp.size != T * K:
        raise ValueError("send_pos must hold T*K entries")
    n_rows = T * K if n_rows is None else n_rows
    msg_bytes = quant_msg_bytes(H) if msg_bytes is None else msg_bytes
    if msgs is None:
        msgs = np.zeros((n_rows, msg_bytes), np.uint8)
    sm = None if smooth is None else _c(smooth, np.float32)
    E = 0 if sm is None else sm.shape[0]
    re = None if route_expert is None else _c(route_expert, np.int32).reshape(-1)
    _check(lib.oracle_dispatch_quant(T, K, H, _p(x), _p(sm), E, _p(re), _p(sp), n_rows, msg_bytes,
                                     _p(msgs)), "oracle_dispatch_quant")
    return msgs


def group_quant(msgs, recv_pos, H):
    """int8 messages [n_msgs, msg_bytes] -> (x_q [n,H] int8 as uint8, scales [n] fp32)
    (oracle_group_quant)."""
    lib = _load()
    m = _c(msgs, np.uint8)
    n_msgs, mb = m.shape
    rp = _c(recv_pos, np.int32).reshape(-1)
    xq = np.zeros((rp.size, H), np.uint8)
    sc = np.zeros(rp.size, np.float32)
    _check(lib.oracle_group_quant(rp.size, H, mb, _p(rp), n_msgs, _p(m), _p(xq), _p(sc)),
           "oracle_group_quant")
    return xq, sc


def weight_rows(plan, R, E, B):
    """Weight row per instance [R, E] under B prefetch slots (oracle_weight_rows)."""
    lib = _load()
    ic = _c(plan["inst_count"], np.int32).reshape(-1)
    ie = _c(plan["inst_expert"], np.int32).reshape(-1)
    out = np.zeros((R, E), np.int32)
    _check(lib.oracle_weight_rows(R, E, B, _p(ic), _p(ie), _p(out)), "oracle_weight_rows")
    return out


def plan_dedup(plan, R, S, K, m):
    """Per-destination dedup maps of rank m from the global plan
    (oracle_plan_dedup): dpack_pos [S*K], dsend_count [R], drecv_pos [S*K],
    drecv_count [R]."""
    lib = _load()
    C = S * K
    rd = _c(plan["route_dest"], np.int32).reshape(-1)
    rs = _c(plan["route_slot"], np.int32).reshape(-1)
    out = dict(dpack_pos=np.zeros(C, np.int32), dsend_count=np.zeros(R, np.int32),
               drecv_pos=np.zeros(C, np.int32), drecv_count=np.zeros(R, np.int32))
    _check(lib.oracle_plan_dedup(R, S, K, m, _p(rd), _p(rs), _p(out["dpack_pos"]),
                                 _p(out["dsend_count"]), _p(out["drecv_pos"]),
                                 _p(out["drecv_count"])), "oracle_plan_dedup")
    return out


def bf16_from_float(a):
    """fp32 -> bf16 round-to-nearest-even (the oracle's own conversion)."""
    lib = _load()
    a = _c(a, np.float32)
    out = np.zeros(a.shape, np.uint16)
    lib.oracle_bf16_from_float(_p(a), _p(out), a.size)
    return out


def float_from_fp16(a):
    lib = _load()
    a = _c(a, np.uint16)
    out = np.zeros(a.shape, np.float32)
    lib.oracle_float_from_fp16(_p(a), _p(out), a.size)
    return out


def chain(x_all, plans, scores_all, expert_fn):
    """Whole chain over every logical rank for small workloads.

    x_all [R,S,H] bf16; plans[r] = plan(..., m=r); scores_all [R,S,K];
    expert_fn(dest, grouped_rows, plan_of_dest) -> expert output rows
    (bf16, same shape). Returns per-rank dicts with send_buf, recv_raw,
    recv_grouped, y_grouped, y_ret, out_bf16, out_f32.

    The source-major arrival buffer of rank d is the concatenation, over
    sources in ascending order, of each source's send segment for d; the
    return path is the exact inverse (the alltoall a multi-GPU run would
    perform, done here with plain numpy slicing).
    """
    R, S, H = x_all.shape
    K = scores_all.shape[2]
    res = [dict() for _ in range(R)]
    seg = []
    for r in range(R):
        p = plans[r]
        res[r]["send_buf"] = pack(x_all[r], p["send_pos"], K)
        off = np.concatenate([[0], np.cumsum(p["send_count"])])
        seg.append(off)
    for d in range(R):
        parts = [res[src]["send_buf"][seg[src][d]:seg[src][d + 1]] for src in range(R)]
        raw = np.concatenate(parts, axis=0)
        res[d]["recv_raw"] = raw
        res[d]["recv_grouped"] = group(raw, plans[d]["recv_pos"])
        yg = expert_fn(d, res[d]["recv_grouped"], plans[d])
        res[d]["y_grouped"] = yg
        res[d]["y_arrival"] = ungroup(yg, plans[d]["recv_pos"])   # back to arrival order
    for src in range(R):
        parts = []
        for d in range(R):
            roff = np.concatenate([[0], np.cumsum(plans[d]["recv_count"])])
            parts.append(res[d]["y_arrival"][roff[src]:roff[src + 1]])
        y_ret = np.concatenate(parts, axis=0)
        res[src]["y_ret"] = y_ret
        ob, of = combine(y_ret, plans[src]["send_pos"], scores_all[src])
        res[src]["out_bf16"] = ob
        res[src]["out_f32"] = of
    return res
