"""Pins of the oracle's plan against things other than itself.

The plan's target is the invariant of the "MoonEP" technical overview
(architecture section): every rank processes exactly S*K routed rows however
skewed the router is, by placing temporary copies of hot experts on other
ranks.
"""
import numpy as np
import pytest

from plan_checks import check_plan, waterfill


def _random_ids(rng, R, E, S, K, skew):
    w = np.exp(-skew * np.log(np.arange(E) + 1.0))
    w = w / w.sum()
    ids = np.empty((R * S, K), np.int32)
    for g in range(R * S):
        ids[g] = rng.choice(E, K, replace=False, p=w)
    return ids


def test_hand_worked_vector(orc):
    # R=2, E=4, S=2, K=2, C=4. Routes f = g*K+k:
    #   f: 0  1  2  3  4  5  6  7
    #   e: 0  1  1  0  0  2  1  3
    # home(e) = floor(e*2/4): e0,e1 -> rank 0; e2,e3 -> rank 1. L = [6, 2].
    # (e,f) order: f0 f3 f4 | f1 f2 f6 | f5 | f7.
    # Rank 0 keeps f0 f3 f4 f1 at slots 0..3; excess f2, f6 (in that order).
    # Rank 1 keeps f5, f7 at slots 0, 1 and takes f2, f6 at slots 2, 3.
    ids = np.array([[0, 1], [1, 0], [0, 2], [1, 3]], np.int32)
    p0 = orc.plan(ids, 2, 4, 2, 2, m=0)
    assert p0["expert_count"].tolist() == [3, 3, 1, 1]
    assert p0["rank_load"].tolist() == [6, 2]
    assert p0["route_dest"].tolist() == [0, 0, 1, 0, 0, 1, 1, 1]
    assert p0["route_slot"].tolist() == [0, 3, 2, 1, 2, 0, 3, 1]
    # rank 0: e0 (3 rows), e1 (1 row); rank 1: e2, e3, then copy of e1 (2 rows)
    assert p0["inst_count"].tolist() == [2, 3]
    assert p0["inst_expert"].tolist() == [[0, 1, -1, -1], [2, 3, 1, -1]]
    assert p0["inst_cu"].tolist() == [[0, 3, 4, 4, 4], [0, 1, 2, 4, 4]]
    assert p0["inst_gid_base"].tolist() == [0, 2, 5]
    # rank 0 sends f0(0,0) f3(0,1) f1(0,3) f2(1,2)
    assert p0["send_pos"].tolist() == [0, 2, 3, 1]
    assert p0["send_count"].tolist() == [3, 1]
    # rank 0 slots hold f0 f3 f4 f1 from sources 0 0 1 0
    assert p0["recv_pos"].tolist() == [0, 1, 3, 2]
    assert p0["recv_count"].tolist() == [3, 1]
    p1 = orc.plan(ids, 2, 4, 2, 2, m=1)
    # rank 1 sends f4(0,2) f5(1,0) f7(1,1) f6(1,3); indexed by local route
    assert p1["send_pos"].tolist() == [0, 1, 3, 2]
    assert p1["send_count"].tolist() == [1, 3]
    # rank 1 slots hold f5 f7 f2 f6 from sources 1 1 0 1
    assert p1["recv_pos"].tolist() == [1, 2, 0, 3]
    assert p1["recv_count"].tolist() == [1, 3]


@pytest.mark.parametrize("seed", range(300))
def test_matches_waterfill_random_tiny(orc, seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 6))
    E = int(rng.integers(1, 21))
    K = int(rng.integers(1, min(E, 4) + 1))
    S = int(rng.integers(1, 9))
    ids = _random_ids(rng, R, E, S, K, skew=float(rng.uniform(0, 3)))
    m = int(rng.integers(0, R))
    p = orc.plan(ids, R, E, S, K, m=m)
    d, s = waterfill(ids, R, E, S, K)
    assert np.array_equal(p["route_dest"], d)
    assert np.array_equal(p["route_slot"], s)
    check_plan(ids, R, E, S, K, m, p)


def test_balanced_routing_has_no_copies(orc):
    # Every rank's experts receive exactly C routes: nothing spills, and each
    # rank's slots are a stable sort of its routes by expert.
    R, E, S, K = 4, 8, 16, 2
    rng = np.random.default_rng(7)
    ids = np.empty((R * S, K), np.int32)
    for g in range(R * S):
        # each token picks one expert of each half of some rank pair: keep
        # per-expert counts equal by cycling
        ids[g] = [(2 * g) % E, (2 * g + 1) % E]
    rng.shuffle(ids.reshape(-1))  # shuffle keeps per-expert counts
    flat = ids.reshape(-1)
    # make each token's ids distinct again is not needed for the plan
    cnt = np.bincount(flat, minlength=E)
    assert np.all(cnt == R * S * K // E)
    p = orc.plan(ids, R, E, S, K, m=0)
    C = S * K
    assert p["rank_load"].tolist() == [C] * R
    home = (np.arange(E) * R) // E
    assert np.all(p["route_dest"] == home[flat])
    for r in range(R):
        mine = np.nonzero(home[flat] == r)[0]
        order = mine[np.argsort(flat[mine], kind="stable")]
        assert np.array_equal(p["route_slot"][order], np.arange(C))
    assert p["inst_count"].tolist() == [E // R] * R


def test_all_routes_on_one_expert(orc):
    # K=1 and every token picks expert e0: the home rank keeps the first C
    # routes, and each other rank u takes C rows of e0 in ascending u.
    R, E, S, K = 4, 8, 5, 1
    e0 = 5
    ids = np.full((R * S, K), e0, np.int32)
    p = orc.plan(ids, R, E, S, K, m=2)
    C = S * K
    h = e0 * R // E
    f = np.arange(R * C)
    others = [u for u in range(R) if u != h]
    exp_dest = np.where(f < C, h, np.array(others)[np.minimum(f // C - 1, R - 2)])
    exp_slot = np.where(f < C, f, f % C)
    # native rows of other ranks: 0, so their slots start at 0
    assert np.array_equal(p["route_dest"], exp_dest)
    assert np.array_equal(p["route_slot"], exp_slot)
    for u in others:
        n_nat = sum(1 for e in range(E) if e * R // E == u)
        assert p["inst_count"][u] == n_nat + 1
        assert p["inst_expert"][u, n_nat] == e0
        assert np.all(p["inst_cu"][u, : n_nat + 1] == 0)  # zero-row natives kept
    check_plan(ids, R, E, S, K, 2, p)


def test_single_rank_is_stable_sort(orc):
    R, E, S, K = 1, 6, 9, 3
    rng = np.random.default_rng(3)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(S)]).astype(np.int32)
    p = orc.plan(ids, R, E, S, K, m=0)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.all(p["route_dest"] == 0)
    assert np.array_equal(p["route_slot"][order], np.arange(S * K))
    assert np.array_equal(p["recv_pos"], np.arange(S * K))
    assert np.array_equal(np.argsort(p["send_pos"]), order)


@pytest.mark.parametrize("R,E", [(4, 4), (6, 3), (8, 5), (5, 1)])
def test_few_experts_per_rank(orc, R, E):
    # E <= R: some ranks host no native expert at all; they are filled
    # entirely with copies.
    rng = np.random.default_rng(R * 10 + E)
    S, K = 7, 1
    ids = rng.integers(0, E, size=(R * S, K)).astype(np.int32)
    for m in range(R):
        p = orc.plan(ids, R, E, S, K, m=m)
        check_plan(ids, R, E, S, K, m, p)
        d, s = waterfill(ids, R, E, S, K)
        assert np.array_equal(p["route_dest"], d)
        assert np.array_equal(p["route_slot"], s)


def test_every_rank_view_is_consistent(orc):
    # The global part of the plan does not depend on which rank asks.
    rng = np.random.default_rng(11)
    R, E, S, K = 5, 12, 6, 3
    ids = _random_ids(rng, R, E, S, K, skew=2.0)
    ps = [orc.plan(ids, R, E, S, K, m=m) for m in range(R)]
    for m in range(1, R):
        for k in ("route_dest", "route_slot", "inst_count", "inst_expert", "inst_cu"):
            assert np.array_equal(ps[0][k], ps[m][k])
    # what m sends to d equals what d receives from m
    for m in range(R):
        for d in range(R):
            assert ps[m]["send_count"][d] == ps[d]["recv_count"][m]


def test_repeated_id_within_token(orc):
    # Not produced by a top-K router, but the (expert, token, k) order still
    # decides: the lower k of a token comes first.
    ids = np.array([[1, 1], [0, 1], [1, 0], [1, 1]], np.int32)
    p = orc.plan(ids, 2, 2, 2, 2, m=0)
    d, s = waterfill(ids, 2, 2, 2, 2)
    assert np.array_equal(p["route_dest"], d)
    assert np.array_equal(p["route_slot"], s)
    check_plan(ids, 2, 2, 2, 2, 0, p)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_workload_plans(orc, name):
    import synth
    d = synth.make_routing(name)
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    for m in sorted({0, R - 1}):
        p = orc.plan(d["topk_ids"], R, E, S, K, m=m)
        check_plan(d["topk_ids"], R, E, S, K, m, p)
    if name == "tiny":
        dd, ss = waterfill(d["topk_ids"], R, E, S, K)
        assert np.array_equal(p["route_dest"], dd)
        assert np.array_equal(p["route_slot"], ss)


def test_rejects_bad_arguments(orc):
    ids = np.zeros((4, 2), np.int32)
    with pytest.raises(orc.OracleError):
        orc.plan(ids, 2, 1, 2, 2)        # K > E
    with pytest.raises(orc.OracleError):
        orc.plan(ids, 2, 4, 2, 2, m=2)   # m out of range
    with pytest.raises(orc.OracleError):
        orc.plan(ids + 9, 2, 4, 2, 2)    # id out of range


def test_scale_checks_accept_oracle_and_catch_a_swap(orc):
    # the checks the maximum-size GPU plan test relies on (the plan rule in
    # vectorised form for every route, the send/arrival permutations), run
    # here on the oracle's plan of the same skewed routing at a small size;
    # a planted swap of two routes' slots must fail them
    import torch
    from test_gpu_plan_max import check_plan_at_scale, skewed_ids
    R, E, S, K, m = 8, 256, 2048, 8, 5
    ids = skewed_ids(R, S, seed=11)
    p = orc.plan(ids.astype(np.int32), R, E, S, K, m=m)
    tp = {k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in p.items()}
    tids = torch.from_numpy(ids.astype(np.int32))
    L = check_plan_at_scale(tids, R, E, S, K, m, tp)
    assert int(L.max()) > S * K
    bad = {k: v.clone() for k, v in tp.items()}
    f = torch.nonzero(bad["route_dest"].reshape(-1) == m).reshape(-1)[:2]
    sl = bad["route_slot"].reshape(-1)
    sl[f[0]], sl[f[1]] = sl[f[1]].clone(), sl[f[0]].clone()
    with pytest.raises(AssertionError):
        check_plan_at_scale(tids, R, E, S, K, m, bad)
