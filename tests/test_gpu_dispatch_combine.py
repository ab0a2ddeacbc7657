"""GPU parity of mep_dispatch (pack, grouping) and mep_combine.

Pack and grouping are bit-exact against the oracle. Combine computes the
same fp32 operations in the same k order as the oracle (each product and
each partial sum rounded on its own, from +0), so both of its outputs are
asserted bit-exact. The stated tolerance (bf16 output within 1 bf16 ulp, fp32
output within 1e-6 relative to the larger of |reference| and the sum of
|score * y| over the token's routes) is checked beside it.
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
    assert np.array_equal(gb, rb), ctx
    assert np.array_equal(gf.view(np.uint32), rf.view(np.uint32)), ctx
    # only the bf16 output requested
    ob2, _ = cba.combine(dev(y), dev(sp), dev(sc), out_bf16=True, out_f32=False)
    torch.cuda.synchronize()
    assert np.array_equal(host(ob2), gb), ctx
    return gb, gf, rb, rf


def test_combine_subnormal_rows(orc):
    # expert rows of bf16 subnormals and tiny scores: products and partial
    # sums in the fp32 subnormal range, taken exactly as the oracle takes them
    require_gpu()
    rng = np.random.default_rng(23)
    T, K, H = 24, 4, 64
    y = (rng.integers(0, 0x80, (T * K, H)) | (rng.integers(0, 2, (T * K, H)) << 15)).astype(np.uint16)
    y[::5] = synth.bf16_normal(rng, (len(y[::5]), H))  # some normal rows beside them
    sp = rng.permutation(T * K).astype(np.int32)
    sc = synth.make_scores(rng, T, K)
    sc[::3, 1] = np.float32(2.0 ** -20)
    _check_combine(orc, y, sp, sc, "subnormal rows")


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


def test_large_skew_whole(orc):
    # S=8192 rows of H=7168 for rank 0 of the R=64 plan (4,194,304 routes),
    # in the benchmark's launch configuration. A few sampled rows are
    # checked first (a fast first failure); then every row of the pack, the
    # grouping and both combine outputs is compared with the oracle.
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
    sbh = host(sb)
    del sb
    for s in rng.choice(S, 64, replace=False):
        for k in range(K):
            assert np.array_equal(sbh[p["send_pos"][s * K + k]], d["x"][s])
    want = orc.pack(d["x"], p["send_pos"], K)
    assert np.array_equal(sbh, want)
    del sbh, want
    note("group large_skew")
    _, rg = cba.dispatch(K, recv_raw=dev(d["recv_raw"]), recv_pos=dev(p["recv_pos"]))
    torch.cuda.synchronize()
    rgh = host(rg)
    del rg
    assert np.array_equal(rgh, orc.group(d["recv_raw"], p["recv_pos"]))
    del rgh
    _check_combine(orc, d["y_ret"], p["send_pos"], d["scores"][0], "large_skew")


def test_combine_order_vectors(orc):
    # vectors whose result changes under any other order or rounding (an
    # fp64 or reversed-order or pairwise sum, a fused multiply-add): the
    # kernels give the oracle's bits, on the unrolled path (K = 4, 2) and the
    # generic one (K = 20), with rows of a ragged vector count
    require_gpu()

    def rows(vals, H):
        bits = (np.array(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return np.repeat(bits[:, None], H, axis=1)

    H = 72
    y = rows([1.0, 2.0 ** -24, 2.0 ** -24, -1.0], H)
    _check_combine(orc, y, np.arange(4, dtype=np.int32), np.ones((1, 4), np.float32),
                   "forward k order")
    y = rows([1.0, 1.0 + 2.0 ** -7], H)
    sc = np.array([[1.0, 1.0 + 2.0 ** -23]], np.float32)
    gb, gf, _, _ = _check_combine(orc, y, np.array([0, 1], np.int32), sc, "product rounding")
    assert np.all(gf == np.float32(2.0 + 2.0 ** -7)) and np.all(gb == 0x4000)
    # K = 20 (generic kernel): the forward-order vector padded with zero
    # rows and skipped routes
    y = rows([1.0, 2.0 ** -24, 2.0 ** -24, -1.0, 0.0], H)
    sp = np.full(20, -1, np.int32)
    sp[[0, 5, 11, 19]] = [0, 1, 2, 3]
    sp[[1, 2]] = 4
    gb, gf, _, _ = _check_combine(orc, y, sp, np.ones((1, 20), np.float32), "generic K=20")
    assert np.all(gf == 0.0)


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


def test_row_kernels_random_shapes(orc):
    # twenty-four seeded (T, K, H) with random skip rates: pack and grouping
    # bit-exact, both combine outputs bit-exact
    torch = require_gpu()
    import combine_balancing_amd as cba
    shapes = np.random.default_rng(20261206)
    for case in range(24):
        T = int(shapes.integers(1, 301))
        K = int(shapes.integers(1, 25))
        H = 8 * int(shapes.integers(1, 2049))
        skip = float(shapes.choice([0.0, 0.1, 0.5]))
        rng = np.random.default_rng(case)
        x = synth.bf16_normal(rng, (T, H))
        sp = rng.permutation(T * K).astype(np.int32)
        sp[rng.random(T * K) < skip] = -1
        note(f"row kernels random case {case}: T={T} K={K} H={H} skip={skip}")
        sb, _ = cba.dispatch(K, x=dev(x), send_pos=dev(sp))
        torch.cuda.synchronize()
        assert np.array_equal(host(sb), orc.pack(x, sp, K)), f"pack case {case}"
        raw = synth.bf16_normal(rng, (T * K, H))
        rp = rng.permutation(T * K).astype(np.int32)
        _, rg = cba.dispatch(K, recv_raw=dev(raw), recv_pos=dev(rp))
        torch.cuda.synchronize()
        assert np.array_equal(host(rg), orc.group(raw, rp)), f"group case {case}"
        sc = rng.standard_normal((T, K)).astype(np.float32)
        _check_combine(orc, raw, sp, sc, f"random case {case} T={T} K={K} H={H}")


def test_short_buffers_bound_the_maps(orc):
    # a map naming rows past the end of its buffer (a plan map paired with a
    # dedup-sized buffer): the pack skips stores past send_buf's rows and the
    # grouping leaves a row untouched when its source is past recv_raw's rows
    torch = require_gpu()
    import combine_balancing_amd as cba
    rng = np.random.default_rng(77)
    T, K, H = 40, 4, 136
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    n_short = T * K // 3
    note("pack into a short send buffer")
    sb = torch.zeros(n_short, H, dtype=torch.bfloat16, device="cuda")
    cba.dispatch(K, x=dev(x), send_pos=dev(sp), send_buf=sb)
    torch.cuda.synchronize()
    assert np.array_equal(host(sb), orc.pack(x, sp, K)[:n_short])
    raw = synth.bf16_normal(rng, (T * K, H))
    rp = rng.permutation(T * K).astype(np.int32)
    note("group from a short arrival buffer")
    rg = torch.zeros(T * K, H, dtype=torch.bfloat16, device="cuda")
    cba.dispatch(K, recv_raw=dev(raw[:n_short]), recv_pos=dev(rp), recv_grouped=rg)
    torch.cuda.synchronize()
    want = orc.group(raw, rp)
    want[rp >= n_short] = 0
    assert np.array_equal(host(rg), want)


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
