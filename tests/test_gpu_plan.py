"""GPU parity of mep_plan against the oracle (bit-exact on every output)."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu
from plan_checks import check_plan

pytestmark = pytest.mark.gpu

KEYS = ["expert_count", "rank_load", "route_dest", "route_slot", "inst_count",
        "inst_expert", "inst_cu", "inst_gid_base", "send_pos", "send_count",
        "recv_pos", "recv_count"]


def _gpu_plan(ids, R, E, S, K, m):
    import combine_balancing_amd as cba
    torch = require_gpu()
    out = cba.plan(dev(np.asarray(ids, np.int32).reshape(-1)), R, E, S, K, my_rank=m)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _assert_same(ref, got, ctx):
    for k in KEYS:
        a = np.asarray(ref[k]).reshape(-1)
        b = np.asarray(got[k]).reshape(-1)
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0]
            raise AssertionError(f"{ctx}: {k} differs at {bad[:8]} "
                                 f"oracle={a[bad[:8]]} gpu={b[bad[:8]]}")


def _rand_ids(rng, R, E, S, K, skew):
    w = np.exp(-skew * np.log(np.arange(E) + 1.0))
    w /= w.sum()
    # Gumbel top-K: distinct ids per token drawn with weights w, in blocks
    # of tokens so that large cases stay small in memory
    out = np.empty((R * S, K), np.int32)
    step = 8192
    for t0 in range(0, R * S, step):
        g = -(rng.gumbel(size=(min(step, R * S - t0), E)) + np.log(w))
        top = np.argpartition(g, K - 1, axis=1)[:, :K] if K < E else np.tile(np.arange(E), (g.shape[0], 1))
        order = np.argsort(np.take_along_axis(g, top, 1), axis=1, kind="stable")
        out[t0:t0 + g.shape[0]] = np.take_along_axis(top, order, 1)
    return out


@pytest.mark.parametrize("name", ["tiny", "small", "dsv3", "large_skew"])
def test_plan_workloads(orc, name):
    require_gpu()
    d = synth.make_routing(name)
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    ranks = sorted({0, R // 2, R - 1})
    for m in ranks:
        note(f"plan {name} R={R} E={E} S={S} K={K} m={m}")
        got = _gpu_plan(d["topk_ids"], R, E, S, K, m)
        ref = orc.plan(d["topk_ids"], R, E, S, K, m=m)
        _assert_same(ref, got, f"{name} m={m}")
    if name in ("tiny", "small"):
        check_plan(d["topk_ids"], R, E, S, K, ranks[-1], got)


# Shapes whose tables fit one work-group's LDS beside the route tables run
# the one-launch form (plan_fused); E near 1000 runs plan_global and
# plan_routes. Both forms are covered with staged ids (chunks up to 2048
# routes) and ids read from global memory, with 8- and 10-bit keys; the
# fused form in 512-thread groups (more than 256 short chunks) by the
# imbalance sweep, the case below and some of the random shapes.
CASES = [
    # (R, E, S, K, skew): ragged chunks, E <= R, one rank, one expert per rank
    (1, 1, 5, 1, 0.0), (1, 7, 300, 3, 1.0), (2, 2, 3, 2, 0.0), (3, 50, 700, 3, 2.0),
    (4, 4, 129, 1, 3.0), (6, 3, 200, 1, 1.0), (5, 1, 64, 1, 0.0), (16, 64, 333, 4, 1.5),
    (64, 256, 40, 8, 1.0), (7, 1024, 150, 16, 0.5), (33, 100, 77, 5, 2.5),
    (128, 1000, 20, 8, 1.0), (1024, 1024, 3, 2, 1.0), (2, 1024, 5000, 2, 3.0),
    # two-launch form, chunks above 2048 routes (ids read from global
    # memory) and 10-bit keys in the wave multi-split
    (64, 1024, 2560, 8, 1.0),
    # one-launch form with experts above 256 (10-bit keys): staged ids, and
    # 4096-route chunks read from global memory
    (8, 384, 1024, 8, 1.0), (64, 300, 2048, 16, 1.0),
    # five chunks per source, the last one ragged
    (8, 64, 1149, 4, 1.5),
    # more chunks than CUs, short ones: the fused form in 512-thread groups
    (300, 128, 125, 8, 1.0), (300, 300, 125, 8, 1.0),
    # more than 512 ranks: one chunk per source rank, at 524,288 and 240,000
    # routes
    (1024, 512, 64, 8, 1.0), (600, 256, 100, 4, 2.0),
]


@pytest.mark.parametrize("R,E,S,K,skew", CASES)
def test_plan_shapes_and_edges(orc, R, E, S, K, skew):
    require_gpu()
    rng = np.random.default_rng(R * 7919 + E * 31 + S)
    ids = _rand_ids(rng, R, E, S, K, skew)
    for m in sorted({0, R - 1, int(rng.integers(0, R))}):
        note(f"plan case R={R} E={E} S={S} K={K} m={m}")
        got = _gpu_plan(ids, R, E, S, K, m)
        ref = orc.plan(ids, R, E, S, K, m=m)
        _assert_same(ref, got, f"R={R} E={E} S={S} K={K} m={m}")


def test_plan_all_on_one_expert(orc):
    require_gpu()
    R, E, S, K = 8, 32, 1000, 1
    ids = np.full((R * S, K), 13, np.int32)
    for m in (0, 3, 7):
        note(f"plan one-expert m={m}")
        _assert_same(orc.plan(ids, R, E, S, K, m=m), _gpu_plan(ids, R, E, S, K, m), "one expert")


def test_plan_is_deterministic():
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_routing("dsv3")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    ids = dev(d["topk_ids"].reshape(-1))
    note("plan determinism dsv3")
    a = cba.plan(ids, R, E, S, K, my_rank=3)
    b = cba.plan(ids, R, E, S, K, my_rank=3)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


def test_plan_without_route_maps(orc):
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_routing("small")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    note("plan small without route maps")
    out = cba.plan(dev(d["topk_ids"].reshape(-1)), R, E, S, K, my_rank=1, with_routes=False)
    torch.cuda.synchronize()
    ref = orc.plan(d["topk_ids"], R, E, S, K, m=1)
    for k in KEYS:
        if k in ("route_dest", "route_slot"):
            continue
        assert np.array_equal(host(out[k]).reshape(-1), ref[k].reshape(-1)), k


def test_plan_rejects_bad_arguments():
    require_gpu()
    import combine_balancing_amd as cba
    from combine_balancing_amd import _binding as B
    import torch
    ids = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MepError):
        cba.plan(ids, 2, 4, 4, 2, my_rank=2)
    ws = cba.plan_workspace(2, 4, 4, 2)
    with pytest.raises(B.MepError):
        cba.plan(ids, 2, 4, 4, 2, my_rank=0, workspace=ws[:16])


@pytest.mark.parametrize("target", [0.2, 1.0, 10.0, 20.0])
def test_plan_skew_sweep(orc, target):
    # the imbalance sweep's shape (R=8, E=384, S=8192, K=8) at every point the
    # benchmark times: every plan output bit-exact
    require_gpu()
    d = synth.make_sweep_routing(target)
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    for m in (0, 5):
        note(f"plan sweep maxvio={target} m={m}")
        got = _gpu_plan(d["topk_ids"], R, E, S, K, m)
        ref = orc.plan(d["topk_ids"], R, E, S, K, m=m)
        _assert_same(ref, got, f"sweep {target} m={m}")


@pytest.mark.parametrize("name", ["tiny", "small", "dsv3", "large_skew"])
def test_plan_weight_rows(orc, name):
    # the prefetch-slot table for B = 0, 3 (inference) and E/R (training),
    # from the GPU plan, against the oracle's on the oracle plan
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_routing(name)
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    note(f"plan weight rows {name}")
    p = cba.plan(dev(d["topk_ids"].reshape(-1)), R, E, S, K, my_rank=0, with_routes=False)
    ref = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    for slots in (0, 3, max(1, E // R)):
        w = cba.plan_weight_rows(p, R, E, slots)
        torch.cuda.synchronize()
        assert np.array_equal(host(w), orc.weight_rows(ref, R, E, slots)), slots


def test_plan_random_shapes(orc):
    """Forty seeded shapes across both plan forms (E up to 1024, R up to 96,
    ragged chunks, skewed and flat routing), each at one random rank."""
    require_gpu()
    shapes = np.random.default_rng(20261204)
    for case in range(40):
        R = int(shapes.integers(1, 97))
        E = int(shapes.integers(1, 1025))
        K = int(shapes.integers(1, min(E, 16) + 1))
        S = min(int(shapes.integers(1, max(2, 300000 // (R * K)))), 2000)
        skew = float(shapes.choice([0.0, 1.0, 2.5]))
        m = int(shapes.integers(0, R))
        ids = _rand_ids(np.random.default_rng(case), R, E, S, K, skew)
        note(f"plan random case {case}: R={R} E={E} S={S} K={K} skew={skew} m={m}")
        _assert_same(orc.plan(ids, R, E, S, K, m=m), _gpu_plan(ids, R, E, S, K, m),
                     f"case {case} R={R} E={E} S={S} K={K} m={m}")
