"""Seeded synthetic inputs for the balanced expert-parallel MoE hot path.

This module is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark. It draws inputs only: router logits and the
top-K selection that stands in for a trained router, bf16 hidden rows, EPLB
tables and pruning thresholds. It holds none of the method's arithmetic (no
planning, remapping, pruning, dispatch or combine).

bf16 values are produced by truncating float32 draws to their upper 16 bits
(round toward zero). That is input generation, not the rounding the combine
step performs.

Workloads (names and sizes follow the five synthetic configurations the
method's benchmark description calls for):

  tiny        R=4  E=16  S=64   K=2 H=128   bias -1.0*ln(e+1)
  small       R=8  E=64  S=1024 K=4 H=2048  bias -1.2*ln(e+1)
  dsv3        R=8  E=256 S=4096 K=8 H=7168  bias N(0,0.5^2), +2.0 on 8 hot experts
  large_skew  R=64 E=256 S=8192 K=8 H=7168  bias -1.0*ln(e+1), +4.0 on expert 0
  eplb        E=512 world_size=384 place_per_rank=2 F=9 BS=512 K=8 H=7168

Draw order per workload: bias, logits (top-K ids and scores), hidden rows,
then stand-in buffers. Seeds 1..5 in the order above.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(R=4, E=16, S=64, K=2, H=128, seed=1),
    "small": dict(R=8, E=64, S=1024, K=4, H=2048, seed=2),
    "dsv3": dict(R=8, E=256, S=4096, K=8, H=7168, seed=3),
    "large_skew": dict(R=64, E=256, S=8192, K=8, H=7168, seed=4),
    "eplb": dict(E=512, world_size=384, place_per_rank=2, F=9, BS=512, K=8,
                 H=7168, n_active=448, seed=5),
}

PLAN_WORKLOADS = ("tiny", "small", "dsv3", "large_skew")

_ROW_CHUNK = 65536  # router rows drawn per call, bounds peak host memory


def bf16_from_f32_trunc(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) by truncation."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 (uint16 bits) rows with values ~N(0,1)."""
    return bf16_from_f32_trunc(rng.standard_normal(shape, dtype=np.float32))


def _topk_desc(logits: np.ndarray, K: int) -> np.ndarray:
    """Top-K column ids per row, in descending logit order, ties to lower id.

    Equivalent to a stable descending argsort truncated to K columns.
    """
    n, E = logits.shape
    if K == E:
        part = np.broadcast_to(np.arange(E), (n, E)).copy()
    else:
        part = np.argpartition(-logits, K - 1, axis=1)[:, :K]
    vals = np.take_along_axis(logits, part, axis=1)
    # lexsort: last key is primary -> sort by -value, then by id
    order = np.lexsort((part, -vals), axis=1)
    ids = np.take_along_axis(part, order, axis=1)
    if K < E:
        # argpartition is only exact when the K-th and (K+1)-th values differ
        kth = np.take_along_axis(logits, ids[:, -1:], axis=1)[:, 0]
        masked = logits.copy()
        np.put_along_axis(masked, ids, -np.inf, axis=1)
        nxt = masked.max(axis=1)
        tie = np.nonzero(nxt >= kth)[0]
        for i in tie:  # fall back to a stable full sort for tied rows
            ids[i] = np.argsort(-logits[i], kind="stable")[:K]
    return ids.astype(np.int32)


def _softmax_f32(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float32)
    e = np.exp(v - v.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _route(rng: np.random.Generator, n_rows: int, E: int, K: int,
           bias: np.ndarray):
    """Router stand-in: logits N(0,1)+bias, top-K ids, softmax scores."""
    ids = np.empty((n_rows, K), np.int32)
    scores = np.empty((n_rows, K), np.float32)
    for r0 in range(0, n_rows, _ROW_CHUNK):
        r1 = min(n_rows, r0 + _ROW_CHUNK)
        lg = rng.standard_normal((r1 - r0, E), dtype=np.float32) + bias
        top = _topk_desc(lg, K)
        ids[r0:r1] = top
        scores[r0:r1] = _softmax_f32(np.take_along_axis(lg, top, axis=1))
    return ids, scores


def _bias(name: str, rng: np.random.Generator, E: int) -> np.ndarray:
    e = np.arange(E, dtype=np.float64)
    if name == "tiny":
        b = -1.0 * np.log(e + 1)
    elif name == "small":
        b = -1.2 * np.log(e + 1)
    elif name == "dsv3":
        b = rng.normal(0.0, 0.5, E)
        hot = rng.choice(E, 8, replace=False)
        b[hot] += 2.0
    elif name == "large_skew":
        b = -1.0 * np.log(e + 1)
        b[0] += 4.0
    else:
        raise KeyError(name)
    return b.astype(np.float32)


def make_routing(name: str, seed: int | None = None):
    """Global routing table of a plan workload.

    Returns dict with topk_ids int32 [R,S,K] and scores fp32 [R,S,K], plus the
    rng positioned after the routing draws (for hidden rows).
    """
    c = WORKLOADS[name]
    rng = np.random.default_rng(c["seed"] if seed is None else seed)
    R, E, S, K = c["R"], c["E"], c["S"], c["K"]
    bias = _bias(name, rng, E)
    ids, scores = _route(rng, R * S, E, K, bias)
    return dict(topk_ids=ids.reshape(R, S, K), scores=scores.reshape(R, S, K),
                rng=rng, **{k: c[k] for k in ("R", "E", "S", "K", "H")})


def make_plan_inputs(name: str, seed: int | None = None, *, rank: int = 0,
                     all_ranks_x: bool | None = None, stand_ins: bool = True):
    """Inputs for plan + dispatch + combine on one workload.

    tiny/small: hidden rows for every rank (x_all [R,S,H]) so the whole
    dispatch -> expert -> combine chain can be replayed across logical ranks.
    dsv3/large_skew: this rank's rows x [S,H] plus seeded stand-ins for the
    received rows (recv_raw [C,H]) and the returned expert outputs
    (y_ret [C,H]).
    """
    d = make_routing(name, seed)
    rng = d.pop("rng")
    R, S, K, H = d["R"], d["S"], d["K"], d["H"]
    C = S * K
    if all_ranks_x is None:
        all_ranks_x = name in ("tiny", "small")
    if all_ranks_x:
        d["x_all"] = bf16_normal(rng, (R, S, H))
        d["x"] = d["x_all"][rank]
    else:
        d["x"] = bf16_normal(rng, (S, H))
        if stand_ins:
            d["recv_raw"] = bf16_normal(rng, (C, H))
            d["y_ret"] = bf16_normal(rng, (C, H))
    d["rank"] = rank
    d["C"] = C
    return d


def make_eplb_inputs(seed: int | None = None, *, with_x: bool = True):
    """EPLB remap + prune workload (and the rows it then dispatches)."""
    c = WORKLOADS["eplb"]
    rng = np.random.default_rng(c["seed"] if seed is None else seed)
    E, F, BS, K, H = c["E"], c["F"], c["BS"], c["K"], c["H"]
    ws, ppr = c["world_size"], c["place_per_rank"]
    n_inst = ws * ppr
    table = np.empty((E, F), np.int32)
    table[:, 0] = rng.integers(1, F, size=E)  # instance count in [1, F-1]
    for e in range(E):
        table[e, 1:] = rng.choice(n_inst, F - 1, replace=False)
    lg = rng.standard_normal((BS, E), dtype=np.float32)
    ids = _topk_desc(lg, K)
    sc = _softmax_f32(np.take_along_axis(lg, ids, axis=1))
    scales = bf16_from_f32_trunc(sc)
    thr = rng.uniform(0.0, 0.2, K).astype(np.float32)
    active = np.zeros(BS, np.uint8)
    active[: c["n_active"]] = 1
    d = dict(expert_ids=ids, eplb_table=table, expert_scales=scales,
             pruning_threshold=thr, active_mask=active, E=E, F=F, BS=BS, K=K,
             H=H, world_size=ws, place_per_rank=ppr)
    if with_x:
        d["x"] = bf16_normal(rng, (BS, H))
    return d


def make_scores(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    """fp32 combine weights: softmax of N(0,1) draws, sorted descending."""
    v = -np.sort(-rng.standard_normal((T, K), dtype=np.float32), axis=1)
    return _softmax_f32(v)


# ------------------------------------------------------------ skew sweep
# The pages' comparison benchmark: EP=8 ranks, S=8192 tokens per rank, E=384
# experts, K=8, H=7168, imbalance (maxvio) 0.2, 1, 10 and 20 from a shared
# routing seed. maxvio there is read at expert granularity (a rank-level
# maxvio cannot exceed R-1 = 7): max_e cnt[e] / (N/E) - 1, with N = R*S*K.
SWEEP = dict(R=8, E=384, S=8192, K=8, H=7168, seed=6)
SWEEP_TARGETS = (0.2, 1.0, 10.0, 20.0)


def expert_maxvio(ids: np.ndarray, E: int) -> float:
    cnt = np.bincount(np.asarray(ids).reshape(-1), minlength=E)
    return float(cnt.max()) / (cnt.sum() / E) - 1.0


def _sweep_alpha(target: float, E: int, K: int, seed: int, n_cal: int = 16384) -> float:
    """Strength of a -alpha*ln(e+1) router bias giving expert maxvio ~target,
    by bisection on a fixed calibration sample of logits."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n_cal, E), dtype=np.float32)
    base = -np.log(np.arange(E, dtype=np.float64) + 1.0).astype(np.float32)
    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        mv = expert_maxvio(_topk_desc(z + np.float32(mid) * base, K), E)
        if mv < target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def make_sweep_routing(target: float):
    """Routing table [R,S,K] of the skew sweep at one maxvio target."""
    c = SWEEP
    R, E, S, K = c["R"], c["E"], c["S"], c["K"]
    alpha = _sweep_alpha(target, E, K, c["seed"] * 1000 + int(round(target * 10)))
    rng = np.random.default_rng(c["seed"])
    bias = (np.float32(alpha) * -np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)
    ids, scores = _route(rng, R * S, E, K, bias)
    return dict(topk_ids=ids.reshape(R, S, K), scores=scores.reshape(R, S, K), alpha=alpha,
                maxvio_expert=expert_maxvio(ids, E), rng=rng, **{k: c[k] for k in ("R", "E", "S", "K", "H")})
