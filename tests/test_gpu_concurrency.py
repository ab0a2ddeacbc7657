"""The library keeps no state between calls (mep.h conventions): calls on
two streams at once, each with its own buffers, give what they give alone.

Two different plans, then two packs, groupings and combines, are enqueued
alternately on two streams (default priority) several times over, and
every output is compared with the oracle bit for bit.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu
from test_gpu_plan import KEYS, _assert_same, _rand_ids

pytestmark = pytest.mark.gpu

REPEATS = 4


def _cases():
    a = synth.make_plan_inputs("small")
    rng = np.random.default_rng(91)
    R, E, S, K, H = 16, 128, 2000, 6, 1024
    ids = _rand_ids(rng, R, E, S, K, 1.5)
    b = dict(topk_ids=ids.reshape(R, S, K), R=R, E=E, S=S, K=K, H=H,
             x=synth.bf16_normal(rng, (S, H)), scores=synth.make_scores(rng, S, K))
    return [(a["topk_ids"], a["R"], a["E"], a["S"], a["K"], a["H"], a["x"], a["scores"][2], 2),
            (b["topk_ids"], R, E, S, K, H, b["x"], b["scores"], 5)]


def test_two_streams_plan_dispatch_combine(orc):
    torch = require_gpu()
    import combine_balancing_amd as cba
    cases = _cases()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    main = torch.cuda.current_stream()
    st = []
    for ids, R, E, S, K, H, x, sc, m in cases:
        C = S * K
        rng = np.random.default_rng(R + S)
        raw = synth.bf16_normal(rng, (C, H))
        st.append(dict(ids=dev(np.asarray(ids, np.int32).reshape(-1)), ws=cba.plan_workspace(R, E, S, K),
                       out=cba.plan_outputs(R, E, S, K), x=dev(x), raw=dev(raw), sc=dev(sc),
                       send=torch.zeros(C, H, dtype=torch.int16, device="cuda"),
                       grouped=torch.zeros(C, H, dtype=torch.int16, device="cuda"),
                       ob=torch.empty(S, H, dtype=torch.bfloat16, device="cuda"),
                       of=torch.empty(S, H, dtype=torch.float32, device="cuda"),
                       raw_np=raw))
    for s in streams:
        s.wait_stream(main)  # inputs were written on the main stream
    for rep in range(REPEATS):
        note(f"two-stream plans, repeat {rep}")
        for (ids, R, E, S, K, H, x, sc, m), b, s in zip(cases, st, streams):
            cba.plan(b["ids"], R, E, S, K, my_rank=m, workspace=b["ws"], out=b["out"], stream=s)
        note(f"two-stream pack, group, combine, repeat {rep}")
        for (ids, R, E, S, K, H, x, sc, m), b, s in zip(cases, st, streams):
            o = b["out"]
            cba.dispatch(K, x=b["x"], send_pos=o["send_pos"], send_buf=b["send"],
                         recv_raw=b["raw"], recv_pos=o["recv_pos"], recv_grouped=b["grouped"],
                         stream=s)
            cba.combine(b["send"], o["send_pos"], b["sc"], out_bf16=b["ob"], out_f32=b["of"],
                        stream=s)
    torch.cuda.synchronize()
    for (ids, R, E, S, K, H, x, sc, m), b in zip(cases, st):
        ref = orc.plan(ids, R, E, S, K, m=m)
        _assert_same(ref, {k: host(v) for k, v in b["out"].items()}, f"R={R} S={S}")
        send = orc.pack(x, ref["send_pos"], K)
        assert np.array_equal(host(b["send"]).view(np.uint16), send)
        assert np.array_equal(host(b["grouped"]).view(np.uint16),
                              orc.group(b["raw_np"], ref["recv_pos"]))
        ob, of = orc.combine(send, ref["send_pos"], sc)
        assert np.array_equal(host(b["ob"]).view(np.uint16), ob)
        assert np.array_equal(host(b["of"]).view(np.uint32), of.view(np.uint32))
