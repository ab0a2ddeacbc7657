"""GPU check of mep_plan_noalloc (the plan with its workspace in the
library's static device array) against mep_plan, called through the C ABI.

Two calls in a row, the second on a smaller plan: every output equals
mep_plan's on the same inputs, bit for bit, so the array's leftovers from
the first call change nothing. A size beyond the array is refused.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, note, require_gpu

pytestmark = pytest.mark.gpu

KEYS = ["expert_count", "rank_load", "route_dest", "route_slot", "inst_count",
        "inst_expert", "inst_cu", "inst_gid_base", "send_pos", "send_count",
        "recv_pos", "recv_count"]


def _call(fn, R, E, S, K, m, ids, out, *ws):
    from combine_balancing_amd import _binding as B
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    rc = fn(R, E, S, K, m, ids.data_ptr(), *ws, *[ptr(out[k]) for k in KEYS], stream)
    assert rc == B.MEP_OK, B.lib().mep_status_str(rc)


def _both(R, E, S, K, m, ids_np):
    torch = require_gpu()
    import combine_balancing_amd as cba
    from combine_balancing_amd import _binding as B
    ids = dev(ids_np.reshape(-1))
    ref = cba.plan_outputs(R, E, S, K)
    got = cba.plan_outputs(R, E, S, K)
    for t in got.values():
        t.fill_(-7)
    ws = cba.plan_workspace(R, E, S, K)
    _call(B.lib().mep_plan, R, E, S, K, m, ids, ref, ws.data_ptr(), ws.numel())
    _call(B.lib().mep_plan_noalloc, R, E, S, K, m, ids, got)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(ref[k], got[k]), k


def test_noalloc_plan_matches_plan_twice():
    require_gpu()
    d = synth.make_routing("large_skew")
    note("mep_plan_noalloc large_skew (R=64 E=256 S=8192 K=8) m=5")
    _both(d["R"], d["E"], d["S"], d["K"], 5, d["topk_ids"])
    d = synth.make_routing("dsv3")
    note("mep_plan_noalloc dsv3 (R=8 E=256 S=4096 K=8) m=0, after a larger plan")
    _both(d["R"], d["E"], d["S"], d["K"], 0, d["topk_ids"])
    d = synth.make_routing("tiny")
    note("mep_plan_noalloc tiny m=3, after two larger plans")
    _both(d["R"], d["E"], d["S"], d["K"], 3, d["topk_ids"])


def test_noalloc_plan_refuses_sizes_beyond_the_array():
    torch = require_gpu()
    import combine_balancing_amd as cba
    from combine_balancing_amd import _binding as B
    R, E, S, K = 1024, 1024, 4, 2
    assert B.lib().mep_plan_workspace_size(R, E, S, K) > B.MEP_PLAN_NOALLOC_SCRATCH_BYTES
    ids = torch.zeros(R * S * K, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MepError) as e:
        cba.plan_noalloc(ids, R, E, S, K)
    assert e.value.code == B.MEP_ERR_SHAPE
