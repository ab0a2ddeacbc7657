"""GPU parity of mep_plan_dedup (per-destination token dedup) against the
oracle, bit-exact, and the dedup dispatch chain against the plain one."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

KEYS = ["dpack_pos", "dsend_count", "drecv_pos", "drecv_count"]


@pytest.mark.parametrize("name", ["tiny", "small", "dsv3", "large_skew"])
def test_dedup_maps(orc, name):
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_routing(name)
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    note(f"dedup maps {name}: plan")
    p = cba.plan(dev(d["topk_ids"].reshape(-1)), R, E, S, K, my_rank=0)
    ref_plan = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    for m in sorted({0, R // 2, R - 1}):
        note(f"dedup maps {name} m={m}")
        got = cba.plan_dedup(p, R, S, K, m)
        torch.cuda.synchronize()
        ref = orc.plan_dedup(ref_plan, R, S, K, m)
        for k in KEYS:
            assert np.array_equal(host(got[k]), ref[k]), (k, m)


@pytest.mark.parametrize("R,E,S,K", [(2, 4, 1500, 3), (5, 9, 2047, 2), (64, 64, 40, 8),
                                     (1, 4, 100, 2), (3, 3, 1025, 1), (4, 32, 1500, 12),
                                     (4, 32, 1500, 20)])
def test_dedup_edge_shapes(orc, R, E, S, K):
    # ragged 1024-token chunks, one rank, the 64-rank limit, K = 1; K = 12
    # (16-byte reads of a token's slots) and K = 20 (more slots than the
    # register-held ones, the rest read one by one)
    torch = require_gpu()
    import combine_balancing_amd as cba
    rng = np.random.default_rng(R * 31 + S)
    g = rng.gumbel(size=(R * S, E)) - 1.5 * np.log(np.arange(E) + 1.0)
    ids = np.argsort(-g, axis=1, kind="stable")[:, :K].astype(np.int32)
    note(f"dedup edge R={R} E={E} S={S} K={K}")
    p = cba.plan(dev(ids.reshape(-1)), R, E, S, K, my_rank=0)
    ref_plan = orc.plan(ids, R, E, S, K, m=0)
    for m in sorted({0, R - 1}):
        got = cba.plan_dedup(p, R, S, K, m)
        torch.cuda.synchronize()
        ref = orc.plan_dedup(ref_plan, R, S, K, m)
        for k in KEYS:
            assert np.array_equal(host(got[k]), ref[k]), (k, m)


@pytest.mark.parametrize("R,E,S,K", [(8, 64, 1500, 8), (4, 32, 1500, 12), (4, 32, 1500, 20)])
def test_dedup_misaligned_route_maps(orc, R, E, S, K):
    # route maps 4 bytes off a 16-byte boundary: the scalar read path must
    # give the same maps as the vector path (K % 4 == 0) and the oracle
    torch = require_gpu()
    import combine_balancing_amd as cba
    rng = np.random.default_rng(77 + K)
    g = rng.gumbel(size=(R * S, E)) - 1.5 * np.log(np.arange(E) + 1.0)
    ids = np.argsort(-g, axis=1, kind="stable")[:, :K].astype(np.int32)
    note(f"dedup misaligned route maps R={R} S={S} K={K}")
    p = cba.plan(dev(ids.reshape(-1)), R, E, S, K, my_rank=0)
    off = {}
    for k in ("route_dest", "route_slot"):
        buf = torch.empty(p[k].numel() + 1, dtype=torch.int32, device="cuda")
        buf[1:] = p[k]
        off[k] = buf[1:]
        assert off[k].data_ptr() % 16 != 0
    ref_plan = orc.plan(ids, R, E, S, K, m=0)
    for m in (0, R - 1):
        got = cba.plan_dedup(off, R, S, K, m)
        aligned = cba.plan_dedup(p, R, S, K, m)
        torch.cuda.synchronize()
        ref = orc.plan_dedup(ref_plan, R, S, K, m)
        for k in KEYS:
            assert np.array_equal(host(got[k]), ref[k]), (k, m)
            assert np.array_equal(host(aligned[k]), ref[k]), (k, m)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_dedup_chain(orc, name):
    # dedup pack -> exchange -> dedup grouping equals every rank's grouped
    # buffer of the plain chain (oracle)
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    ref_plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    ref = orc.chain(d["x_all"], ref_plans, d["scores"],
                    lambda dst, rows, plan: rows)
    note(f"dedup chain {name}")
    p = cba.plan(dev(d["topk_ids"].reshape(-1)), R, E, S, K, my_rank=0)
    dd = [cba.plan_dedup(p, R, S, K, m) for m in range(R)]
    torch.cuda.synchronize()
    counts = [host(q["dsend_count"]) for q in dd]
    sends = []
    for m in range(R):
        buf = torch.zeros(int(counts[m].sum()), H, dtype=torch.bfloat16, device="cuda")
        cba.dispatch(K, x=dev(d["x_all"][m]), send_pos=dd[m]["dpack_pos"], send_buf=buf)
        sends.append(buf)
    off = [np.concatenate([[0], np.cumsum(c)]) for c in counts]
    for r in range(R):
        raw = torch.cat([sends[src][off[src][r]:off[src][r + 1]] for src in range(R)])
        assert raw.shape[0] == host(dd[r]["drecv_count"]).sum()
        _, grouped = cba.dispatch(K, recv_raw=raw, recv_pos=dd[r]["drecv_pos"],
                                  recv_grouped=torch.empty(S * K, H, dtype=torch.bfloat16,
                                                           device="cuda"))
        torch.cuda.synchronize()
        assert np.array_equal(host(grouped), ref[r]["recv_grouped"])


def test_dedup_random_shapes(orc):
    """Twenty seeded shapes (R up to 64, E up to 512, K up to 24, ragged
    1024-token chunks, skewed and flat routing), each at a random rank."""
    torch = require_gpu()
    import combine_balancing_amd as cba
    shapes = np.random.default_rng(20261209)
    for case in range(20):
        R = int(shapes.integers(1, 65))
        E = int(shapes.integers(1, 513))
        K = int(shapes.integers(1, min(E, 24) + 1))
        S = int(shapes.integers(1, max(2, min(3000, 60000 // (R * K)))))
        skew = float(shapes.choice([0.0, 1.5]))
        m = int(shapes.integers(0, R))
        rng = np.random.default_rng(case)
        g = rng.gumbel(size=(R * S, E)) - skew * np.log(np.arange(E) + 1.0)
        ids = np.argsort(-g, axis=1, kind="stable")[:, :K].astype(np.int32)
        note(f"dedup random case {case}: R={R} E={E} S={S} K={K} m={m}")
        p = cba.plan(dev(ids.reshape(-1)), R, E, S, K, my_rank=m)
        ref_plan = orc.plan(ids, R, E, S, K, m=m)
        got = cba.plan_dedup(p, R, S, K, m)
        torch.cuda.synchronize()
        ref = orc.plan_dedup(ref_plan, R, S, K, m)
        for k in KEYS:
            assert np.array_equal(host(got[k]), ref[k]), (case, k)
