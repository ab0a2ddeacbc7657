#!/usr/bin/env python3
"""Benchmark of the balanced expert-parallel MoE hot path on one MI355X.

One step = the whole hot path on synthetic inputs already resident in HBM:
  plan (global plan over the R x S x K routing table, this rank's maps),
  remap + prune (EPLB workload: BS=512, K=8, E=512, world 384),
  pack, receive grouping and combine of one rank's share
  (R=8, E=256, S=4096, K=8, H=7168, bf16 rows).
The headline value is dispatch+combine effective HBM bandwidth: the
algorithmic bytes of pack + group + combine divided by their measured time
(a HIP event pair on the launch stream around the three kernels, mean over
the timed steps). A second set of steps with an event pair around every
kernel gives the per-kernel breakdown and the roofline's kernel time; an
event between two kernels adds a few us of launch gap, so those intervals
run slightly long.

Prints one JSON line. --gpus above 1 is refused: the path runs on one GPU (R is a
logical world size).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
# extra measurements after the headline step, in the order they run
LEGS = ("copy_reference", "graph_step", "combine_add_rmsnorm", "int8_dispatch",
        "dedup_dispatch", "zero_copy", "large_skew", "skew_sweep")
WORKLOAD = "dsv3"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dsv3.json")
# sources the row-moving kernels are compiled from: the stored counter
# figures hold only while these are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "combine_balancing_amd", "csrc", f)
               for f in ("dispatch.hip", "rows.h", "mep_device.h")]
FLUSH_BYTES = 1 << 30


def algorithmic_bytes(S, K, H, out_f32=False):
    """Bytes the method must move, each x row read once (per launch)."""
    C = S * K
    pack = S * H * 2 + C * H * 2 + C * 4
    group = 2 * C * H * 2 + C * 4
    combine = C * H * 2 + 2 * C * 4 + S * H * 2 + (S * H * 4 if out_f32 else 0)
    return dict(pack=pack, group=group, combine=combine)


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def sources_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(kernel):
    """HBM bytes per launch from committed counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        src_hash = sources_sha256()
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != src_hash:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, plan_ref, budget_s=10.0):
    """The oracle (single-threaded C) on the same workload: full passes of
    pack + group + combine of the rank-0 share, repeated until about
    budget_s seconds of host time are spent (at least 3); the median pass
    gives the rate."""
    import oracle
    S, K, H = d["S"], d["K"], d["H"]
    oracle.plan(d["topk_ids"][:1], 1, d["E"], S, K, 0)  # load + warm the library
    b = algorithmic_bytes(S, K, H)
    total = b["pack"] + b["group"] + b["combine"]
    passes = []
    t_start = time.perf_counter()
    while len(passes) < 3 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        oracle.pack(d["x"], plan_ref["send_pos"], K)
        oracle.group(d["recv_raw"], plan_ref["recv_pos"])
        oracle.combine(d["y_ret"], plan_ref["send_pos"], d["scores"][0], want_f32=False)
        passes.append(time.perf_counter() - t0)
    t0 = time.perf_counter()
    oracle.plan(d["topk_ids"], d["R"], d["E"], S, K, 0)
    plan_s = time.perf_counter() - t0
    dt = float(np.median(passes))
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(passes)} full passes of pack+group+combine, {WORKLOAD} rank 0 "
                      f"({total} algorithmic bytes each), median {dt:.3f} s per pass, "
                      f"{time.perf_counter() - t_start:.1f} s in all",
            "plan_s": round(plan_s, 4),
            "routes_per_s_dispatch_combine": round(S * K / dt, 1),
            "routes_per_s_plan": round(d["R"] * S * K / plan_s, 1),
            "host_cpu": cpu_model(),
            "host_cpu_count": os.cpu_count()}


def skew_sweep(torch, cba, synth, steps, flush=None):
    """Plan and dispatch+combine time as router imbalance grows (expert-level
    maxvio 0.2, 1, 10, 20) at R=8, E=384, S=8192, K=8, H=7168, rank 0. The
    received rows and returned expert outputs are seeded stand-ins (their
    content does not affect the time); the routing, hence every index map,
    is the sweep point's own."""
    c = synth.SWEEP
    R, E, S, K, H = c["R"], c["E"], c["S"], c["K"], c["H"]
    C = S * K
    g = torch.Generator(device="cuda")
    g.manual_seed(c["seed"])
    x = torch.randn(S, H, device="cuda", generator=g).to(torch.bfloat16)
    recv_raw = torch.randn(C, H, device="cuda", generator=g).to(torch.bfloat16)
    y_ret = torch.randn(C, H, device="cuda", generator=g).to(torch.bfloat16)
    send_buf = torch.empty(C, H, dtype=torch.bfloat16, device="cuda")
    grouped = torch.empty(C, H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    ws = cba.plan_workspace(R, E, S, K)
    pout = cba.plan_outputs(R, E, S, K)
    b = algorithmic_bytes(S, K, H)
    dc_bytes = b["pack"] + b["group"] + b["combine"]
    stream = torch.cuda.current_stream()
    points = []
    for target in synth.SWEEP_TARGETS:
        d = synth.make_sweep_routing(target)
        ids = _dev(torch, d["topk_ids"].reshape(-1))
        scores = _dev(torch, d["scores"][0])
        times = {"plan": [], "dispatch_combine": []}
        for it in range(steps + 3):
            if flush is not None:
                flush.fill_(it & 0xFF)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            cba.plan(ids, R, E, S, K, my_rank=0, workspace=ws, out=pout)
            ev[1].record(stream)
            cba.dispatch(K, x=x, send_pos=pout["send_pos"], send_buf=send_buf)
            cba.dispatch(K, recv_raw=recv_raw, recv_pos=pout["recv_pos"], recv_grouped=grouped)
            cba.combine(y_ret, pout["send_pos"], scores, out_bf16=out)
            ev[2].record(stream)
            torch.cuda.synchronize()
            if it >= 3:
                times["plan"].append(ev[0].elapsed_time(ev[1]) * 1e3)
                times["dispatch_combine"].append(ev[1].elapsed_time(ev[2]) * 1e3)
        loads = pout["rank_load"].cpu().numpy()
        n_inst = int(pout["inst_gid_base"][-1].item())
        dc = float(np.median(times["dispatch_combine"]))
        points.append({"target_maxvio": target,
                       "expert_maxvio": round(d["maxvio_expert"], 3),
                       "rank_maxvio_native": round(float(loads.max()) / C - 1.0, 3),
                       "instances": n_inst, "redundant_instances": n_inst - E,
                       "plan_us": round(float(np.median(times["plan"])), 2),
                       "dispatch_combine_us": round(dc, 2),
                       "dispatch_combine_GBs": round(dc_bytes / (dc * 1e-6) / 1e9, 1)})
    return {"workload": f"R={R} E={E} S={S} K={K} H={H} bf16, rank 0; maxvio at expert "
                        "granularity (max expert load / mean - 1)", "points": points}


def zero_copy(torch, cba, d, pout, steps, flush=None):
    """The zero-copy pair at the same workload: rank 0 pushes its rows
    straight into the R grouped buffers and pulls the expert outputs back
    from them. On one GPU the R buffers are slices of one [R, C, H]
    allocation standing in for the peers' memory (over xGMI the same kernels
    write and read remote HBM through mapped peer pointers)."""
    R, S, K, H, C = d["R"], d["S"], d["K"], d["H"], d["C"]
    x = _dev(torch, d["x"])
    scores = _dev(torch, d["scores"][0])
    grouped = torch.empty(R, C, H, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    y = torch.randn(R, C, H, device="cuda", generator=g).to(torch.bfloat16)
    gp, yp = cba.peer_table(grouped), cba.peer_table(y)
    rd, rs = pout["route_dest"][:C], pout["route_slot"][:C]
    out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    t = {"push": [], "pull": []}
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        cba.dispatch_to_peers(K, x, rd, rs, gp, C)
        ev[1].record(stream)
        cba.combine_from_peers(yp, C, H, rd, rs, scores, out_bf16=out)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            t["push"].append(ev[0].elapsed_time(ev[1]) * 1e3)
            t["pull"].append(ev[1].elapsed_time(ev[2]) * 1e3)
    us = {k: float(np.mean(v)) for k, v in t.items()}
    row = H * 2
    nb = {"push": S * row + C * row + 2 * C * 4, "pull": C * row + S * row + C * 12}
    del grouped, y
    return {"push_us": round(us["push"], 2), "pull_us": round(us["pull"], 2),
            "push_GBs": round(nb["push"] / (us["push"] * 1e-6) / 1e9, 1),
            "pull_GBs": round(nb["pull"] / (us["pull"] * 1e-6) / 1e9, 1),
            "dispatch_combine_us": round(us["push"] + us["pull"], 2),
            "algorithmic_bytes": nb}


def fused_norm(torch, cba, d, pout, y_ret, scores, steps, flush=None):
    """Combine fused with the residual add and RMSNorm at the same workload
    (rank 0's send map, the same returned expert rows), against the plain
    combine: the fused kernel reads the residual and writes x and y."""
    S, K, H, C = d["S"], d["K"], d["H"], d["C"]
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    res = torch.randn(S, H, device="cuda", generator=g).to(torch.bfloat16)
    gamma = torch.randn(H, device="cuda", generator=g).to(torch.bfloat16)
    x_out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    y_out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(S, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    t = []
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        cba.combine_add_rmsnorm(y_ret, pout["send_pos"], scores, res, gamma, eps=1e-6,
                                x_out=x_out, y_out=y_out, rstd_out=rstd)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            t.append(ev[0].elapsed_time(ev[1]) * 1e3)
    us = float(np.mean(t))
    nb = C * H * 2 + 2 * C * 4 + S * H * 2 + H * 2 + 2 * S * H * 2 + S * 4
    return {"us": round(us, 2), "GBs": round(nb / (us * 1e-6) / 1e9, 1),
            "algorithmic_bytes": nb,
            "outputs": "y bf16 [S,H], x bf16 [S,H], rstd fp32 [S]; eps 1e-6"}


def int8_dispatch(torch, cba, d, pout, steps, flush=None):
    """The pack with int8 dynamic quantization at the same workload (rank 0's
    send map): Align512(Align32(H)+4)-byte messages instead of bf16 rows."""
    S, K, H, C = d["S"], d["K"], d["H"], d["C"]
    x = _dev(torch, d["x"])
    mb = cba.quant_msg_bytes(H)
    msgs = torch.empty(C, mb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    xq = torch.empty(C, H, dtype=torch.int8, device="cuda")
    sc = torch.empty(C, dtype=torch.float32, device="cuda")
    t = {"pack": [], "group": []}
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        cba.dispatch_quant(K, x, pout["send_pos"], send_msgs=msgs)
        ev[1].record(stream)
        if flush is not None:
            # the messages just written would otherwise partly sit in the
            # last-level cache; arrivals come from other GPUs
            flush.fill_((it + 1) & 0xFF)
        # receive side on the same rows (stand-in for the arrival buffer)
        ev[2].record(stream)
        cba.group_quant(msgs, pout["recv_pos"], H, x_q=xq, scales=sc)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            t["pack"].append(ev[0].elapsed_time(ev[1]) * 1e3)
            t["group"].append(ev[2].elapsed_time(ev[3]) * 1e3)
    us = {k: float(np.mean(v)) for k, v in t.items()}
    nb = {"pack": S * H * 2 + C * (H + 4) + C * 4, "group": 2 * C * (H + 4) + C * 4}
    return {"pack_us": round(us["pack"], 2),
            "pack_GBs": round(nb["pack"] / (us["pack"] * 1e-6) / 1e9, 1),
            "group_us": round(us["group"], 2),
            "group_GBs": round(nb["group"] / (us["group"] * 1e-6) / 1e9, 1),
            "algorithmic_bytes": nb, "msg_bytes": mb,
            "bytes_sent_vs_bf16": round(C * mb / (C * H * 2), 4)}


def dedup_dispatch(torch, cba, d, pout, steps, flush=None):
    """Per-destination dedup at the same workload: the dedup maps from the
    plan, the pack of one row per (token, destination), and the grouping
    that fans the arrival rows out to the C grouped slots (the arrival
    buffer here is a stand-in of the dedup arrival count's rows)."""
    R, S, K, H, C = d["R"], d["S"], d["K"], d["H"], d["C"]
    x = _dev(torch, d["x"])
    ws = torch.empty(cba.lib().mep_plan_dedup_workspace_size(R, S, K), dtype=torch.uint8,
                     device="cuda")
    q = cba.plan_dedup(pout, R, S, K, 0, workspace=ws)
    torch.cuda.synchronize()
    n_send = int(q["dsend_count"].sum().item())
    n_arr = int(q["drecv_count"].sum().item())
    send = torch.empty(n_send, H, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    raw = torch.randn(n_arr, H, device="cuda", generator=g).to(torch.bfloat16)
    grouped = torch.empty(C, H, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    t = {"maps": [], "pack": [], "group": []}
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        cba.plan_dedup(pout, R, S, K, 0, workspace=ws, out=q)
        ev[1].record(stream)
        cba.dispatch(K, x=x, send_pos=q["dpack_pos"], send_buf=send)
        ev[2].record(stream)
        cba.dispatch(K, recv_raw=raw, recv_pos=q["drecv_pos"], recv_grouped=grouped)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            for j, k in enumerate(("maps", "pack", "group")):
                t[k].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    us = {k: float(np.mean(v)) for k, v in t.items()}
    row = H * 2
    nb = {"pack": S * row + n_send * row + C * 4, "group": n_arr * row + C * row + C * 4}
    return {"maps_us": round(us["maps"], 2), "pack_us": round(us["pack"], 2),
            "pack_GBs": round(nb["pack"] / (us["pack"] * 1e-6) / 1e9, 1),
            "group_us": round(us["group"], 2),
            "group_GBs": round(nb["group"] / (us["group"] * 1e-6) / 1e9, 1),
            "rows_sent": n_send, "rows_arrived": n_arr, "rows_sent_vs_plain": round(n_send / C, 4),
            "algorithmic_bytes": nb}


def large_skew(torch, cba, synth, steps, flush=None):
    """The large plan with extreme skew (R=64, E=256, S=8192, K=8, H=7168):
    the global plan over all 4,194,304 routes, then rank 0's pack, grouping
    and combine (seeded stand-ins for the received rows and the returned
    expert outputs)."""
    d = synth.make_plan_inputs("large_skew")
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]
    ids = _dev(torch, d["topk_ids"].reshape(-1))
    x, recv_raw, y_ret = _dev(torch, d["x"]), _dev(torch, d["recv_raw"]), _dev(torch, d["y_ret"])
    scores = _dev(torch, d["scores"][0])
    ws = cba.plan_workspace(R, E, S, K)
    pout = cba.plan_outputs(R, E, S, K)
    send_buf = torch.empty(C, H, dtype=torch.int16, device="cuda")
    grouped = torch.empty(C, H, dtype=torch.int16, device="cuda")
    out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    # the plan and the dispatch+combine block, with no events between kernels
    blk = {"plan": [], "dispatch_combine": []}
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        cba.plan(ids, R, E, S, K, my_rank=0, workspace=ws, out=pout)
        ev[1].record(stream)
        cba.dispatch(K, x=x, send_pos=pout["send_pos"], send_buf=send_buf)
        cba.dispatch(K, recv_raw=recv_raw, recv_pos=pout["recv_pos"], recv_grouped=grouped)
        cba.combine(y_ret, pout["send_pos"], scores, out_bf16=out)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            blk["plan"].append(ev[0].elapsed_time(ev[1]) * 1e3)
            blk["dispatch_combine"].append(ev[1].elapsed_time(ev[2]) * 1e3)
    # per-kernel breakdown: an event pair around every kernel
    names = ["plan", "pack", "group", "combine"]
    t = {n: [] for n in names}
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        cba.plan(ids, R, E, S, K, my_rank=0, workspace=ws, out=pout)
        ev[1].record(stream)
        cba.dispatch(K, x=x, send_pos=pout["send_pos"], send_buf=send_buf)
        ev[2].record(stream)
        cba.dispatch(K, recv_raw=recv_raw, recv_pos=pout["recv_pos"], recv_grouped=grouped)
        ev[3].record(stream)
        cba.combine(y_ret, pout["send_pos"], scores, out_bf16=out)
        ev[4].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            for j, n in enumerate(names):
                t[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
    us = {n: float(np.mean(v)) for n, v in t.items()}
    b = algorithmic_bytes(S, K, H)
    plan_us = float(np.mean(blk["plan"]))
    dc = float(np.mean(blk["dispatch_combine"]))
    loads = pout["rank_load"].cpu().numpy()
    n_inst = int(pout["inst_gid_base"][-1].item())
    return {"workload": f"R={R} E={E} S={S} K={K} H={H} bf16, rank 0",
            "plan_us": round(plan_us, 2),
            "routes_per_s_plan": round(R * C / (plan_us * 1e-6), 1),
            "kernel_us_mean": {n: round(v, 2) for n, v in us.items()},
            "dispatch_combine_us": round(dc, 2),
            "dispatch_combine_GBs": round((b["pack"] + b["group"] + b["combine"]) / (dc * 1e-6) / 1e9, 1),
            "maxvio_native": round(float(loads.max()) / C - 1.0, 3),
            "redundant_instances": n_inst - E}


def graph_step(torch, step, steps, flush=None):
    """The headline step captured once in a HIP graph and replayed (the
    library only enqueues: no host sync, allocation or memset inside)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(do_flush=False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(do_flush=False)  # the cache flush stays outside the graph and the timed region
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t = []
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            t.append(ev[0].elapsed_time(ev[1]) * 1e3)
    return {"step_us": round(float(np.mean(t)), 2), "step_us_median": round(float(np.median(t)), 2),
            "what": "plan + remap/prune + pack + group + combine, one graph replay"}


def plan_graph(torch, cba, ids, R, E, S, K, pout, steps, flush=None):
    """The plan alone, captured in a HIP graph through the allocation-free
    entry point (mep_plan_noalloc: no workspace to allocate, nothing to
    clear) and replayed with cold caches. Beside the eager plan_us this
    shows how much of the plan's time is the host enqueueing its launches."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cba.plan_noalloc(ids, R, E, S, K, my_rank=0, out=pout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cba.plan_noalloc(ids, R, E, S, K, my_rank=0, out=pout)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t = []
    for it in range(steps + 3):
        if flush is not None:
            flush.fill_(it & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        if it >= 3:
            t.append(ev[0].elapsed_time(ev[1]) * 1e3)
    return round(float(np.median(t)), 2)


def copy_reference(torch, cba, K, recv_raw, grouped, group_gbs, steps, flush=None):
    """Copy references at the grouping's size, same cold caches: the grouping
    kernel with the identity map (a purely sequential copy) and torch's
    device-to-device copy."""
    C, H = recv_raw.shape
    stream = torch.cuda.current_stream()
    ident = torch.arange(C, dtype=torch.int32, device="cuda")
    refs = {}
    for name, fn in (("identity_grouping", lambda: cba.dispatch(K, recv_raw=recv_raw, recv_pos=ident,
                                                                 recv_grouped=grouped)),
                     ("torch_copy", lambda: grouped.copy_(recv_raw))):
        ct = []
        for it in range(steps + 3):
            if flush is not None:
                flush.fill_(it & 0xFF)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            if it >= 3:
                ct.append(ev[0].elapsed_time(ev[1]) * 1e3)
        cus = float(np.mean(ct))
        refs[name] = {"us": round(cus, 2), "GBs": round(2 * C * H * 2 / (cus * 1e-6) / 1e9, 1)}
    return dict(bytes=2 * C * H * 2, **refs,
                group_rows_vs_identity=round(group_gbs / refs["identity_grouping"]["GBs"], 4))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not write a 1 GiB buffer before each step (caches stay warm)")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated extra legs after the headline step, from: "
                         + ", ".join(LEGS) + " ('none' for the headline step alone)")
    ap.add_argument("--no-skew-sweep", action="store_true", help="drop the skew_sweep leg")
    ap.add_argument("--no-large-skew", action="store_true", help="drop the large_skew leg")
    ap.add_argument("--no-zero-copy", action="store_true", help="drop the zero_copy leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run plain row copies (the library's "
                         "ungroup kernel with the identity map) of the group kernel's "
                         "output size: a known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the hot path is one rank's share "
              "(R is a logical world size); --gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_balancing_amd as cba
    import synth

    torch.cuda.set_device(0)
    cba.lib()
    d = synth.make_plan_inputs(WORKLOAD)
    e = synth.make_eplb_inputs(with_x=False)
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]

    ids = _dev(torch, d["topk_ids"].reshape(-1))
    x = _dev(torch, d["x"])
    recv_raw = _dev(torch, d["recv_raw"])
    y_ret = _dev(torch, d["y_ret"])
    scores = _dev(torch, d["scores"][0])
    ws = cba.plan_workspace(R, E, S, K)
    pout = cba.plan_outputs(R, E, S, K)
    send_buf = torch.empty(C, H, dtype=torch.int16, device="cuda")
    grouped = torch.empty(C, H, dtype=torch.int16, device="cuda")
    out = torch.empty(S, H, dtype=torch.bfloat16, device="cuda")
    e_ids, e_tab = _dev(torch, e["expert_ids"]), _dev(torch, e["eplb_table"])
    e_sc, e_thr = _dev(torch, e["expert_scales"]), _dev(torch, e["pruning_threshold"])
    e_act = _dev(torch, e["active_mask"])
    e_out = dict(balanced_ids=torch.empty(e["BS"], e["K"], dtype=torch.int32, device="cuda"),
                 balanced_mask=torch.empty(e["BS"], e["K"], dtype=torch.uint8, device="cuda"),
                 send_pos=torch.empty(e["BS"] * e["K"], dtype=torch.int32, device="cuda"),
                 send_count=torch.empty(e["world_size"], dtype=torch.int32, device="cuda"))
    stream = torch.cuda.current_stream()

    flush = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    n_step = [0]

    def step(ev=None, do_flush=True, per_kernel=False):
        """One step. With `ev`, events mark the step's start, the end of the
        plan, of remap/prune and of combine; with per_kernel also the ends of
        pack and group. An event between two kernels costs a few us of
        launch gap, so the timed steps leave them out."""
        if flush is not None and do_flush:
            # evict the last-level cache (MALL) and L2 before each step: a
            # step starts with cold caches, as in a model between layers
            n_step[0] += 1
            flush.fill_(n_step[0] & 0xFF)
        if ev is not None:
            ev[0].record(stream)
        cba.plan(ids, R, E, S, K, my_rank=0, workspace=ws, out=pout)
        if ev is not None:
            ev[1].record(stream)
        cba.remap_prune(e_ids, e_tab, e["world_size"], e["place_per_rank"], 0, 0,
                        expert_scales=e_sc, scale_dtype="bf16", pruning_threshold=e_thr,
                        active_mask=e_act, out=e_out)
        if ev is not None:
            ev[2].record(stream)
        cba.dispatch(K, x=x, send_pos=pout["send_pos"], send_buf=send_buf)
        if ev is not None and per_kernel:
            ev[3].record(stream)
        cba.dispatch(K, recv_raw=recv_raw, recv_pos=pout["recv_pos"], recv_grouped=grouped)
        if ev is not None and per_kernel:
            ev[4].record(stream)
        cba.combine(y_ret, pout["send_pos"], scores, out_bf16=out)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps: plan, remap/prune and the dispatch+combine block
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plan_t = [ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs]
    remap_t = [ev[1].elapsed_time(ev[2]) * 1e3 for ev in evs]
    dc_t = [ev[2].elapsed_time(ev[5]) * 1e3 for ev in evs]
    step_us = [ev[0].elapsed_time(ev[5]) * 1e3 for ev in evs]
    # breakdown steps: the same step with an event pair around every kernel
    bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(bevs[i], per_kernel=True)
    torch.cuda.synchronize()
    names = ["plan", "remap_prune", "pack", "group", "combine"]
    per = {n: [] for n in names}
    for ev in bevs:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)  # us
    us = {n: float(np.mean(v)) for n, v in per.items()}
    med = {n: float(np.median(v)) for n, v in per.items()}
    p10 = {n: float(np.percentile(v, 10)) for n, v in per.items()}
    p90 = {n: float(np.percentile(v, 90)) for n, v in per.items()}

    b = algorithmic_bytes(S, K, H)
    dc_bytes = b["pack"] + b["group"] + b["combine"]
    dc_us = float(np.mean(dc_t))
    value = dc_bytes / (dc_us * 1e-6) / 1e9
    group_gbs = b["group"] / (us["group"] * 1e-6) / 1e9

    # correctness spot-check of this run's outputs against the oracle's plan
    # is done by the test suite; here only the plan's balance is reported
    loads = pout["rank_load"].cpu().numpy()
    maxvio_native = float(loads.max()) / C - 1.0

    res = {
        "metric": "dispatch+combine effective HBM bandwidth (pack+group+combine), "
                  "S=4096 K=8 H=7168",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_us)) / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy generator, no dataset)",
        "config": {"workload": "dsv3: R=8 E=256 S=4096 K=8 H=7168 bf16, rank 0; "
                               "plus EPLB remap+prune BS=512 K=8 E=512 world=384",
                   "R": R, "E": E, "S": S, "K": K, "H": H},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "plan_us": round(float(np.mean(plan_t)), 2),
        "remap_prune_us": round(float(np.mean(remap_t)), 2),
        "timing": "value: pack+group+combine as one event interval per timed step (no events "
                  "between the three kernels); kernel_us_*: as many further steps with an event "
                  "pair around every kernel (each interval then holds a few us of event gap)",
        "dispatch_combine_us_median": round(float(np.median(dc_t)), 2),
        "kernel_us_mean": {n: round(v, 2) for n, v in us.items()},
        "kernel_us_median": {n: round(v, 2) for n, v in med.items()},
        "kernel_us_p10": {n: round(v, 2) for n, v in p10.items()},
        "kernel_us_p90": {n: round(v, 2) for n, v in p90.items()},
        "cache_flush_bytes_between_steps": 0 if flush is None else FLUSH_BYTES,
        "dispatch_combine_us": round(dc_us, 2),
        "routes_per_s_dispatch_combine": round(C / (dc_us * 1e-6), 1),
        "routes_per_s_plan": round(R * C / (float(np.mean(plan_t)) * 1e-6), 1),
        "maxvio_native": round(maxvio_native, 4),
        "maxvio_planned": 0.0,
        "algorithmic_bytes": b,
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": "group_rows", "achieved": round(group_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(group_gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("group_rows")},
        # the same figures for each row mover of the step (per-kernel event
        # intervals, algorithmic bytes, HBM peak)
        "kernel_rooflines": {
            kern: {"achieved": round(b[n] / (us[n] * 1e-6) / 1e9, 2),
                   "frac": round(b[n] / (us[n] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes": b[n], "us": round(us[n], 2), "traffic": _traffic(kern)}
            for n, kern in (("pack", "pack_flat"), ("group", "group_rows"),
                            ("combine", "combine_flat"))},
    }
    legs = set() if args.legs == "none" else set(args.legs.split(","))
    unknown = legs - set(LEGS)
    if unknown:
        raise SystemExit(f"unknown legs: {sorted(unknown)}")
    for flag, leg in ((args.no_skew_sweep, "skew_sweep"), (args.no_large_skew, "large_skew"),
                      (args.no_zero_copy, "zero_copy")):
        if flag:
            legs.discard(leg)
    leg_steps = max(5, min(args.steps, 20))
    if "copy_reference" in legs:
        res["copy_reference"] = copy_reference(torch, cba, K, recv_raw, grouped, group_gbs,
                                               steps=leg_steps, flush=flush)
    if "graph_step" in legs:
        res["graph_step"] = graph_step(torch, step, steps=leg_steps, flush=flush)
        res["graph_step"]["plan_us_median"] = plan_graph(torch, cba, ids, R, E, S, K, pout,
                                                         steps=leg_steps, flush=flush)
    if "combine_add_rmsnorm" in legs:
        res["combine_add_rmsnorm"] = fused_norm(torch, cba, d, pout, y_ret, scores,
                                                steps=leg_steps, flush=flush)
    if "int8_dispatch" in legs:
        res["int8_dispatch"] = int8_dispatch(torch, cba, d, pout, steps=leg_steps, flush=flush)
    if "dedup_dispatch" in legs:
        res["dedup_dispatch"] = dedup_dispatch(torch, cba, d, pout, steps=leg_steps, flush=flush)
    if "zero_copy" in legs:
        res["zero_copy"] = zero_copy(torch, cba, d, pout, steps=leg_steps, flush=flush)
    if "large_skew" in legs:
        res["large_skew"] = large_skew(torch, cba, synth, steps=leg_steps, flush=flush)
    if "skew_sweep" in legs:
        res["skew_sweep"] = skew_sweep(torch, cba, synth, steps=leg_steps, flush=flush)
    if args.copy_calibration:
        # a plain copy of known size for scaling the byte counters: the
        # library's own row copy (mep_ungroup with the identity map, so the
        # same one-row-per-work-group request pattern as the grouping; a
        # kernel name of its own, launched nowhere else in a run). torch's
        # device copy may run on a DMA engine, which no kernel counter sees.
        nbytes = C * H * 2
        ident = torch.arange(C, dtype=torch.int32, device="cuda")
        for _ in range(3):
            cba.ungroup(recv_raw, ident, y_arrival=grouped)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = nbytes
        res["copy_calibration_kernel"] = "ungroup_rows (identity map)"
    if not args.no_cpu_baseline:
        import oracle
        plan_ref = oracle.plan(d["topk_ids"], R, E, S, K, 0)
        res["cpu_baseline"] = cpu_baseline(d, plan_ref)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
