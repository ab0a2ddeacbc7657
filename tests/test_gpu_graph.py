"""A whole step captured in a HIP graph and replayed.

Every entry point only enqueues work on the current stream (no host
synchronisation, no allocation, no memset), so one step - plan, remap and
prune, pack, grouping, combine - can be captured once and replayed. Each
replay is compared bit for bit with the eager result on the same inputs;
between replays the inputs change and the program does unrelated eager work
and synchronises.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu


def _step(cba, st):
    cba.plan(st["ids"], st["R"], st["E"], st["S"], st["K"], my_rank=0, workspace=st["ws"],
             out=st["pout"])
    cba.remap_prune(st["e_ids"], st["e_tab"], st["ws_world"], st["ppr"], 0, 0,
                    expert_scales=st["e_sc"], scale_dtype="bf16",
                    pruning_threshold=st["e_thr"], active_mask=st["e_act"], out=st["e_out"])
    cba.dispatch(st["K"], x=st["x"], send_pos=st["pout"]["send_pos"], send_buf=st["send"])
    cba.dispatch(st["K"], recv_raw=st["raw"], recv_pos=st["pout"]["recv_pos"],
                 recv_grouped=st["grouped"])
    cba.combine(st["send"], st["pout"]["send_pos"], st["scores"], out_bf16=st["out"])


def _outputs(st):
    o = {k: host(v) for k, v in st["pout"].items() if v is not None}
    o.update({"e_" + k: host(v) for k, v in st["e_out"].items()})
    o.update(send=host(st["send"]), grouped=host(st["grouped"]), out=host(st["out"]))
    return o


@pytest.mark.parametrize("name", ["small", "dsv3"])
def test_step_graph_replays(orc, name):
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs(name, all_ranks_x=False)
    e = synth.make_eplb_inputs(with_x=False)
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]
    rng = np.random.default_rng(5)
    st = dict(R=R, E=E, S=S, K=K, ids=dev(d["topk_ids"].reshape(-1)), x=dev(d["x"]),
              raw=dev(synth.bf16_normal(rng, (C, H))), scores=dev(d["scores"][0]),
              ws=cba.plan_workspace(R, E, S, K), pout=cba.plan_outputs(R, E, S, K),
              send=torch.zeros(C, H, dtype=torch.int16, device="cuda"),
              grouped=torch.zeros(C, H, dtype=torch.int16, device="cuda"),
              out=torch.zeros(S, H, dtype=torch.bfloat16, device="cuda"),
              e_ids=dev(e["expert_ids"]), e_tab=dev(e["eplb_table"]),
              e_sc=dev(e["expert_scales"]), e_thr=dev(e["pruning_threshold"]),
              e_act=dev(e["active_mask"]), ws_world=e["world_size"], ppr=e["place_per_rank"],
              e_out=dict(balanced_ids=torch.empty(e["BS"], e["K"], dtype=torch.int32, device="cuda"),
                         balanced_mask=torch.empty(e["BS"], e["K"], dtype=torch.uint8, device="cuda"),
                         send_pos=torch.empty(e["BS"] * e["K"], dtype=torch.int32, device="cuda"),
                         send_count=torch.empty(e["world_size"], dtype=torch.int32, device="cuda")))
    note(f"graph {name}: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(cba, st)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(cba, st)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        # new routing and rows for this replay, written into the captured inputs
        d2 = synth.make_plan_inputs(name, seed=100 + rep, all_ranks_x=False)
        st["ids"].copy_(dev(d2["topk_ids"].reshape(-1)))
        st["x"].copy_(dev(d2["x"]))
        st["scores"].copy_(dev(d2["scores"][0]))
        note(f"graph {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(st)
        scratch.add_(1.0)  # unrelated eager work between replays
        _step(cba, st)     # the eager result on the same inputs
        torch.cuda.synchronize()
        want = _outputs(st)
        for k, v in want.items():
            assert np.array_equal(got[k], v), (rep, k)
        # and the replayed plan is the oracle's
        ref = orc.plan(d2["topk_ids"], R, E, S, K, m=0)
        assert np.array_equal(got["send_pos"], ref["send_pos"])
        assert np.array_equal(got["recv_pos"], ref["recv_pos"])


def test_noalloc_plan_graph_replays(orc):
    # the allocation-free plan (its workspace in the library's static array)
    # captured alone in a HIP graph: each replay, on new routing written
    # into the captured input, equals the oracle's plan on every output
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_routing("dsv3")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    ids = dev(d["topk_ids"].reshape(-1))
    out = cba.plan_outputs(R, E, S, K)
    note("graph noalloc plan: warm-up and capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cba.plan_noalloc(ids, R, E, S, K, my_rank=2, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cba.plan_noalloc(ids, R, E, S, K, my_rank=2, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        d2 = synth.make_routing("dsv3", seed=200 + rep)
        ids.copy_(dev(d2["topk_ids"].reshape(-1)))
        note(f"graph noalloc plan: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref = orc.plan(d2["topk_ids"], R, E, S, K, m=2)
        for k, v in ref.items():
            assert np.array_equal(host(out[k]).reshape(-1), v.reshape(-1)), (rep, k)
        # eager work of another entry point between replays
        cba.plan(ids, R, E, S, K, my_rank=0)
        torch.cuda.synchronize()
