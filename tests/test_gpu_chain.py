"""Whole dispatch -> expert -> combine chain over every logical rank, GPU vs
oracle, on the small workloads (every intermediate buffer compared).

The alltoall between logical ranks is emulated with device-to-device slice
copies on one GPU (what RCCL would move between GPUs); the synthetic expert
scales each grouped row by (1 + 0.01 * instance gid) in fp32 and rounds once
to bf16. Everything of the method runs in the library's kernels.
"""
import numpy as np
import pytest

import synth
from gpu_util import bf16_ulp_diff, dev, f32, host, note, require_gpu

pytestmark = pytest.mark.gpu


def _gid_scale(plan, d):
    """fp32 per-slot factors of rank d from its instance table (host)."""
    cu = plan["inst_cu"][d]
    n = plan["inst_count"][d]
    base = plan["inst_gid_base"][d]
    C = cu[-1]
    f = np.empty(C, np.float32)
    for i in range(n):
        f[cu[i]:cu[i + 1]] = np.float32(1.0 + 0.01 * (base + i))
    return f


def _oracle_expert(orc):
    def fn(d, rows, plan):
        prod = f32(rows) * _gid_scale(plan, d)[:, None]
        return orc.bf16_from_float(prod)
    return fn


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_chain(orc, name):
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    ref_plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    ref = orc.chain(d["x_all"], ref_plans, d["scores"], _oracle_expert(orc))

    ids = dev(d["topk_ids"].reshape(-1))
    note(f"chain {name}: plans")
    plans = [cba.plan(ids, R, E, S, K, my_rank=m) for m in range(R)]
    torch.cuda.synchronize()
    hplans = [{k: host(v) for k, v in p.items()} for p in plans]
    for m in range(R):
        for k in ref_plans[m]:
            assert np.array_equal(hplans[m][k].reshape(-1), ref_plans[m][k].reshape(-1)), k

    note(f"chain {name}: pack")
    send = [cba.dispatch(K, x=dev(d["x_all"][m]), send_pos=plans[m]["send_pos"])[0]
            for m in range(R)]
    soff = [np.concatenate([[0], np.cumsum(hp["send_count"])]) for hp in hplans]
    roff = [np.concatenate([[0], np.cumsum(hp["recv_count"])]) for hp in hplans]
    note(f"chain {name}: group + expert")
    y_arrival = []
    for dst in range(R):
        raw = torch.cat([send[src][soff[src][dst]:soff[src][dst + 1]] for src in range(R)])
        _, grouped = cba.dispatch(K, recv_raw=raw, recv_pos=plans[dst]["recv_pos"])
        f = dev(_gid_scale(hplans[dst], dst))
        yg = (grouped.view(torch.bfloat16).float() * f[:, None]).to(torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(raw), ref[dst]["recv_raw"])
        assert np.array_equal(host(grouped), ref[dst]["recv_grouped"])
        assert np.array_equal(host(yg), ref[dst]["y_grouped"])
        # back to arrival order (the expert-side return)
        ya = cba.ungroup(yg, plans[dst]["recv_pos"])
        torch.cuda.synchronize()
        assert np.array_equal(host(ya), ref[dst]["y_arrival"])
        y_arrival.append(ya)
    note(f"chain {name}: combine")
    for src in range(R):
        y_ret = torch.cat([y_arrival[dst][roff[dst][src]:roff[dst][src + 1]]
                           for dst in range(R)])
        ob, of = cba.combine(y_ret, plans[src]["send_pos"], dev(d["scores"][src]),
                             out_bf16=True, out_f32=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(y_ret), ref[src]["y_ret"])
        assert np.all(bf16_ulp_diff(host(ob), ref[src]["out_bf16"]) <= 1)
        rf = ref[src]["out_f32"].astype(np.float64)
        assert np.all(np.abs(host(of).astype(np.float64) - rf) <= 1e-6 * np.abs(rf) + 1e-30)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_zero_copy_chain(orc, name):
    # Every logical rank writes its rows straight into the grouped buffers
    # (slices of one [R, C, H] allocation stand in for the peers' memory):
    # each buffer must equal what pack -> exchange -> group produced; reading
    # the expert outputs in place must give the oracle's combine.
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    C = S * K
    ref_plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    ref = orc.chain(d["x_all"], ref_plans, d["scores"], _oracle_expert(orc))
    note(f"zero-copy chain {name}: plan")
    p = cba.plan(dev(d["topk_ids"].reshape(-1)), R, E, S, K, my_rank=0)
    grouped = torch.zeros(R, C, H, dtype=torch.bfloat16, device="cuda")
    peers = cba.peer_table(grouped)
    note(f"zero-copy chain {name}: push")
    for m in range(R):
        cba.dispatch_to_peers(K, dev(d["x_all"][m]), p["route_dest"][m * C:(m + 1) * C],
                              p["route_slot"][m * C:(m + 1) * C], peers, C)
    torch.cuda.synchronize()
    for r in range(R):
        assert np.array_equal(host(grouped[r]), ref[r]["recv_grouped"])
    y = torch.stack([dev(ref[r]["y_grouped"]).view(torch.bfloat16) for r in range(R)])
    ypeers = cba.peer_table(y)
    note(f"zero-copy chain {name}: pull")
    for m in range(R):
        ob, of = cba.combine_from_peers(ypeers, C, H, p["route_dest"][m * C:(m + 1) * C],
                                        p["route_slot"][m * C:(m + 1) * C],
                                        dev(d["scores"][m]), out_bf16=True, out_f32=True)
        torch.cuda.synchronize()
        assert np.all(bf16_ulp_diff(host(ob), ref[m]["out_bf16"]) <= 1)
        rf = ref[m]["out_f32"].astype(np.float64)
        assert np.all(np.abs(host(of).astype(np.float64) - rf) <= 1e-6 * np.abs(rf) + 1e-30)
        # same fp32 operations in the same k order as the oracle: bit-exact
        assert np.array_equal(host(ob), ref[m]["out_bf16"])
        assert np.array_equal(host(of).view(np.uint32), ref[m]["out_f32"].view(np.uint32))


def test_zero_copy_headline_shape(orc):
    # rank 0 of the R=8, E=256, S=4096, K=8, H=7168 workload: every pushed
    # row lands at its (destination, slot), and the pull equals the oracle's
    # for every token, bit for bit
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs("dsv3", stand_ins=False)
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    rd, rs = dev(p["route_dest"][:C]), dev(p["route_slot"][:C])
    grouped = torch.zeros(R, C, H, dtype=torch.bfloat16, device="cuda")
    note("zero-copy push dsv3")
    cba.dispatch_to_peers(K, dev(d["x"]), rd, rs, cba.peer_table(grouped), C)
    torch.cuda.synchronize()
    g = host(grouped)
    want = orc.push(d["x"], p["route_dest"][:C], p["route_slot"][:C], K, R, C)
    assert np.array_equal(g, want)
    del g, want, grouped
    note("zero-copy pull dsv3")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(123)
    y = torch.randn(R, C, H, device="cuda", generator=gen).to(torch.bfloat16)
    sc = d["scores"][0]
    ob, of = cba.combine_from_peers(cba.peer_table(y), C, H, rd, rs, dev(sc), out_bf16=True,
                                    out_f32=True)
    torch.cuda.synchronize()
    yh = host(y)
    rb, rf = orc.pull_combine(yh, p["route_dest"][:C].reshape(S, K),
                              p["route_slot"][:C].reshape(S, K), sc)
    gb, gf = host(ob), host(of)
    assert np.all(bf16_ulp_diff(gb, rb) <= 1)
    rf64 = rf.astype(np.float64)
    mag = np.abs(rf64).max()
    assert np.all(np.abs(gf.astype(np.float64) - rf64) <= 1e-6 * mag)
    assert np.array_equal(gb, rb)
    assert np.array_equal(gf.view(np.uint32), rf.view(np.uint32))


@pytest.mark.parametrize("T,K,H,R,C", [(3, 2, 65536, 2, 4), (5, 3, 72, 3, 6), (1, 1, 8, 1, 1),
                                       (300, 8, 64, 1024, 4), (50, 20, 136, 1000, 3)])
def test_zero_copy_and_ungroup_edges(orc, T, K, H, R, C):
    # the largest row, ragged vector tails, one rank and one slot, the
    # largest peer table (1024 ranks, staged whole in LDS by the pull) and a
    # generic-K one; routes outside [0,R) x [0,C) are skipped
    torch = require_gpu()
    import combine_balancing_amd as cba
    rng = np.random.default_rng(T * 7 + H)
    x = synth.bf16_normal(rng, (T, H))
    rd = rng.integers(0, R, T * K).astype(np.int32)
    rs = rng.integers(0, C, T * K).astype(np.int32)
    rd[::4] = R  # no such rank
    # one route per (dest, slot): keep the first writer of each slot
    seen = set()
    for f in range(T * K):
        if (rd[f], rs[f]) in seen:
            rd[f] = -1
        seen.add((rd[f], rs[f]))
    note(f"zero-copy edges T={T} K={K} H={H} R={R} C={C}")
    grouped = torch.zeros(R, C, H, dtype=torch.bfloat16, device="cuda")
    cba.dispatch_to_peers(K, dev(x), dev(rd), dev(rs), cba.peer_table(grouped), C)
    torch.cuda.synchronize()
    want = orc.push(x, rd, rs, K, R, C)
    assert np.array_equal(host(grouped), want)
    y = synth.bf16_normal(rng, (R, C, H))
    sc = rng.standard_normal((T, K)).astype(np.float32)
    yd = dev(y).view(torch.bfloat16)  # the peer table holds raw addresses: keep yd alive
    ob, of = cba.combine_from_peers(cba.peer_table(yd), C, H, dev(rd), dev(rs), dev(sc),
                                    out_bf16=True, out_f32=True)
    torch.cuda.synchronize()
    rb, rf = orc.pull_combine(y, rd, rs, sc)
    assert np.array_equal(host(ob), rb) and np.array_equal(host(of), rf)
    n = min(T * K, 16)
    rows = synth.bf16_normal(rng, (n, H))
    rp = rng.permutation(n).astype(np.int32)
    ya = cba.ungroup(dev(rows), dev(rp))
    torch.cuda.synchronize()
    assert np.array_equal(host(ya), orc.ungroup(rows, rp))


def test_zero_copy_random_shapes(orc):
    """Sixteen seeded shapes for the zero-copy push and pull: T up to 200,
    K up to 16, up to 256 ranks, ragged rows, routes outside the buffers and
    repeated (dest, slot) pairs dropped; whole buffers compared."""
    torch = require_gpu()
    import combine_balancing_amd as cba
    shapes = np.random.default_rng(20261210)
    for case in range(16):
        T = int(shapes.integers(1, 201))
        K = int(shapes.integers(1, 17))
        R = int(shapes.integers(1, 257))
        C = int(shapes.integers(1, max(2, 2 * T * K // R + 2)))
        H = 8 * int(shapes.integers(1, max(2, min(1025, 2_000_000 // (8 * R * C)))))
        rng = np.random.default_rng(case)
        x = synth.bf16_normal(rng, (T, H))
        rd = rng.integers(0, R + 1, T * K).astype(np.int32)  # R: no such rank
        rs = rng.integers(0, C, T * K).astype(np.int32)
        seen = set()
        for f in range(T * K):
            if (rd[f], rs[f]) in seen:
                rd[f] = -1
            seen.add((rd[f], rs[f]))
        note(f"zero-copy random case {case}: T={T} K={K} H={H} R={R} C={C}")
        grouped = torch.zeros(R, C, H, dtype=torch.bfloat16, device="cuda")
        cba.dispatch_to_peers(K, dev(x), dev(rd), dev(rs), cba.peer_table(grouped), C)
        torch.cuda.synchronize()
        assert np.array_equal(host(grouped), orc.push(x, rd, rs, K, R, C)), f"case {case}"
        del grouped
        y = synth.bf16_normal(rng, (R, C, H))
        sc = rng.standard_normal((T, K)).astype(np.float32)
        yd = dev(y).view(torch.bfloat16)  # the peer table holds raw addresses: keep yd alive
        ob, of = cba.combine_from_peers(cba.peer_table(yd), C, H, dev(rd), dev(rs), dev(sc),
                                        out_bf16=True, out_f32=True)
        torch.cuda.synchronize()
        rb, rf = orc.pull_combine(y, rd, rs, sc)
        assert np.array_equal(host(ob), rb), f"case {case}"
        assert np.array_equal(host(of).view(np.uint32), rf.view(np.uint32)), f"case {case}"
        del yd
