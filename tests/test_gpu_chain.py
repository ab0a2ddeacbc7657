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
        # back to arrival order: the inverse of grouping is grouping by the
        # inverse permutation
        inv = torch.empty_like(plans[dst]["recv_pos"])
        inv[plans[dst]["recv_pos"].long()] = torch.arange(inv.numel(), dtype=torch.int32,
                                                          device="cuda")
        _, ya = cba.dispatch(K, recv_raw=yg, recv_pos=inv)
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
