"""GPU parity of mep_dispatch (pack, grouping) and mep_combine.

Pack and grouping are bit-exact against the oracle. Combine: bf16 output
within 1 bf16 ulp and fp32 output within 1e-6 relative (to the larger of
|reference| and the sum of |score * y| over the token's routes) of the
oracle, which uses the same k order and rounding.
"""
import numpy as np
import pytest

import synth
from gpu_util import bf16_ulp_diff, dev, f32, host, note, require_gpu

pytestmark = pytest.mark.gpu


def _combine_tol_ok(ref32, got32, y, send_pos, scores):
    T, K = scores.shape
    H = y.shape[1]
    sp = send_pos.reshape(T, K)
    mag = np.zeros((T, H), np.float64)
    for k in range(K):
        ok = sp[:, k] >= 0
        rows = f32(y[np.maximum(sp[:, k], 0)]).astype(np.float64)
        mag += np.where(ok[:, None], np.abs(scores[:, k:k + 1].astype(np.float64) * rows), 0.0)
    bound = 1e-6 * np.maximum(np.abs(ref32.astype(np.float64)), mag)
    return np.abs(got32.astype(np.float64) - ref32.astype(np.float64)) <= bound


def _check_combine(orc, y, sp, sc, ctx):
    torch = require_gpu()
    import combine_balancing_amd as cba
    note(f"combine {ctx}")
    ob, of = cba.combine(dev(y), dev(sp), dev(sc), out_bf16=True, out_f32=True)
    torch.cuda.synchronize()
    gb, gf = host(ob), host(of)
    rb, rf = orc.combine(y, sp, sc)
    assert np.all(bf16_ulp_diff(gb, rb) <= 1), ctx
    assert np.all(_combine_tol_ok(rf, gf, y, sp, sc)), ctx
    # only the bf16 output requested
    ob2, _ = cba.combine(dev(y), dev(sp), dev(sc), out_bf16=True, out_f32=False)
    torch.cuda.synchronize()
    assert np.array_equal(host(ob2), gb), ctx
    return gb, gf, rb, rf


@pytest.fixture(scope="module")
def dsv3(orc):
    require_gpu()
    d = synth.make_plan_inputs("dsv3")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    d["plan"] = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    return d


def test_pack_group_combine_dsv3(orc, dsv3):
    # the headline shape (R=8, E=256, S=4096, K=8, H=7168), whole outputs
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = dsv3
    K, C = d["K"], d["C"]
    p = d["plan"]
    note("pack dsv3")
    sb, _ = cba.dispatch(K, x=dev(d["x"]), send_pos=dev(p["send_pos"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(sb), orc.pack(d["x"], p["send_pos"], K))
    note("group dsv3")
    _, rg = cba.dispatch(K, recv_raw=dev(d["recv_raw"]), recv_pos=dev(p["recv_pos"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(rg), orc.group(d["recv_raw"], p["recv_pos"]))
    _check_combine(orc, d["y_ret"], p["send_pos"], d["scores"][0], "dsv3")


def test_dsv3_identity_roundtrip(orc, dsv3):
    # combine(pack(x)) with identity experts and scores summing to one
    # returns x (the fp32 sum is within a few fp32 ulps of x)
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = dsv3
    note("identity roundtrip dsv3")
    x = dev(d["x"])
    sp = dev(d["plan"]["send_pos"])
    sb, _ = cba.dispatch(d["K"], x=x, send_pos=sp)
    ob, _ = cba.combine(sb, sp, dev(d["scores"][0]))
    torch.cuda.synchronize()
    assert np.all(bf16_ulp_diff(host(ob), d["x"]) <= 1)


def test_large_skew_sampled(orc):
    # S=8192 rows of H=7168 for one rank of the R=64 plan, in the same launch
    # configuration as the benchmark; outputs checked on sampled rows
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_plan_inputs("large_skew")
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]
    note("plan large_skew m=0 (oracle)")
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    rng = np.random.default_rng(4040)
    note("pack large_skew")
    sb, _ = cba.dispatch(K, x=dev(d["x"]), send_pos=dev(p["send_pos"]))
    torch.cuda.synchronize()
    rows = rng.choice(S, 512, replace=False)
    sbh = host(sb)
    for s in rows:
        for k in range(K):
            assert np.array_equal(sbh[p["send_pos"][s * K + k]], d["x"][s])
    note("group large_skew")
    _, rg = cba.dispatch(K, recv_raw=dev(d["recv_raw"]), recv_pos=dev(p["recv_pos"]))
    torch.cuda.synchronize()
    t = rng.choice(C, 4096, replace=False)
    assert np.array_equal(host(rg)[t], orc.group(d["recv_raw"], p["recv_pos"][t]))
    note("combine large_skew")
    ob, of = cba.combine(dev(d["y_ret"]), dev(p["send_pos"]), dev(d["scores"][0]),
                         out_bf16=True, out_f32=True)
    torch.cuda.synchronize()
    tok = np.sort(rng.choice(S, 256, replace=False))
    sp_s = p["send_pos"].reshape(S, K)[tok].reshape(-1)
    sc_s = d["scores"][0][tok]
    rb, rf = orc.combine(d["y_ret"], sp_s, sc_s)
    assert np.all(bf16_ulp_diff(host(ob)[tok], rb) <= 1)
    assert np.all(_combine_tol_ok(rf, host(of)[tok], d["y_ret"], sp_s, sc_s))


def test_eplb_pack_after_remap(orc):
    # remap + prune, then pack the kept routes of BS=512 tokens of H=7168
    torch = require_gpu()
    import combine_balancing_amd as cba
    d = synth.make_eplb_inputs()
    for mode in (0, 1):
        note(f"eplb remap+pack mode={mode}")
        ref = orc.remap_prune(d["expert_ids"], d["eplb_table"], d["world_size"],
                              d["place_per_rank"], 0, mode, expert_scales=d["expert_scales"],
                              pruning_threshold=d["pruning_threshold"],
                              active_mask=d["active_mask"])
        out = cba.remap_prune(dev(d["expert_ids"]), dev(d["eplb_table"]), d["world_size"],
                              d["place_per_rank"], 0, mode,
                              expert_scales=dev(d["expert_scales"]), scale_dtype="bf16",
                              pruning_threshold=dev(d["pruning_threshold"]),
                              active_mask=dev(d["active_mask"]))
        sb, _ = cba.dispatch(d["K"], x=dev(d["x"]), send_pos=out["send_pos"])
        torch.cuda.synchronize()
        n_kept = int((ref["send_pos"] >= 0).sum())
        want = orc.pack(d["x"], ref["send_pos"], d["K"])
        got = host(sb)
        assert np.array_equal(got[:n_kept], want[:n_kept])
        assert not got[n_kept:].any()   # rows past the kept ones untouched (zeros)
        # combine over the kept routes with identity experts
        sc = np.where(ref["balanced_mask"] > 0, 0.25, 0.0).astype(np.float32)
        _check_combine(orc, want[:max(n_kept, 1)], ref["send_pos"], sc, f"eplb mode={mode}")


@pytest.mark.parametrize("T,K,H", [(1, 1, 8), (5, 3, 8), (37, 4, 136), (64, 8, 1032),
                                   (130, 2, 4096), (33, 6, 16384), (9, 20, 512), (3, 64, 64),
                                   (3, 2, 65536), (2, 7, 65528)])
def test_row_kernels_odd_shapes(orc, T, K, H):
    # ragged vector tails (H/8 not a multiple of 64), K beyond the unrolled
    # combine instances, negative and out-of-range entries skipped
    torch = require_gpu()
    import combine_balancing_amd as cba
    rng = np.random.default_rng(T * 1000 + K * 10 + H)
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    sp[rng.random(T * K) < 0.2] = -1
    note(f"pack T={T} K={K} H={H}")
    sb, _ = cba.dispatch(K, x=dev(x), send_pos=dev(sp))
    torch.cuda.synchronize()
    assert np.array_equal(host(sb), orc.pack(x, sp, K))
    n = T * K
    raw = synth.bf16_normal(rng, (n, H))
    rp = rng.permutation(n).astype(np.int32)
    note(f"group n={n} H={H}")
    _, rg = cba.dispatch(K, recv_raw=dev(raw), recv_pos=dev(rp))
    torch.cuda.synchronize()
    assert np.array_equal(host(rg), orc.group(raw, rp))
    sc = (rng.standard_normal((T, K)).astype(np.float32))
    _check_combine(orc, raw, sp, sc, f"T={T} K={K} H={H}")


def test_empty_inputs():
    torch = require_gpu()
    import combine_balancing_amd as cba
    from combine_balancing_amd import _binding as B
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    sp = torch.zeros(0, dtype=torch.int32, device="cuda")
    note("empty dispatch/combine")
    sb, _ = cba.dispatch(4, x=x, send_pos=sp)
    assert sb.shape == (0, 64)
    y = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    ob, _ = cba.combine(y, sp, torch.zeros(0, 4, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert ob.shape == (0, 64)
    with pytest.raises(B.MepError):
        cba.dispatch(4, x=torch.zeros(2, 12, dtype=torch.bfloat16, device="cuda"),
                     send_pos=torch.zeros(8, dtype=torch.int32, device="cuda"))
