"""Pins of the oracle's pack, receive grouping and combine.

Pack and grouping are row permutations ("MoonEP" technical overview,
architecture section: tokens land at their final place grouped by expert on
the receiving rank), pinned against numpy's own indexing. Combine is the
score-weighted K-way sum, pinned by closed forms and by an fp64 evaluation
within the error bound of a K-term fp32 sum.
"""
import numpy as np
import pytest

import synth

U = 2.0 ** -24  # unit roundoff of fp32


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_nearest_even(x):
    """Independent RNE: compare distances to the two bracketing bf16 values
    in fp64 and break ties on the even mantissa."""
    x = np.asarray(x, np.float32)
    lo = (x.view(np.uint32) >> 16).astype(np.uint32)          # toward zero
    hi = lo + 1
    vlo = (lo << 16).view(np.float32).astype(np.float64)
    vhi = (hi << 16).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dlo = np.abs(xd - vlo)
    dhi = np.abs(vhi - xd)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo & 1 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_rne_against_distance_rule(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000, dtype=np.float32),
        rng.standard_normal(2000, dtype=np.float32) * np.float32(1e30),
        # exact ties: bf16 value plus half an ulp
        ((rng.integers(0x3f00, 0x4100, 4000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    fin = np.isfinite(x) & (np.abs(x) < np.float32(3.38e38))
    got = orc.bf16_from_float(x[fin])
    assert np.array_equal(got, _bf16_nearest_even(x[fin]))


def test_rne_specials(orc):
    # IEEE conversion: a NaN stays a NaN of the same sign, even when its
    # payload lies only in the 16 bits that are cut off (truncating those
    # would turn it into an infinity); infinities and signed zeros are kept;
    # values past the largest bf16 by half an ulp or more round to infinity.
    nan_bits = np.array([0x7F800001, 0xFF800001, 0x7F80FFFF, 0x7FC00000, 0xFFFFFFFF,
                         0x7FBFFFFF], np.uint32)
    got = orc.bf16_from_float(nan_bits.view(np.float32)).astype(np.uint32)
    assert np.all((got & 0x7F80) == 0x7F80) and np.all((got & 0x007F) != 0)
    assert np.array_equal(got >> 15, nan_bits >> 31)
    big = np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)
    assert list(orc.bf16_from_float(big)) == [0x7F80, 0xFF80, 0x0000, 0x8000]
    # largest bf16 is 0x7F7F; 0x7F7F8000 is the tie above it (odd mantissa:
    # rounds up, to infinity), 0x7F7F7FFF stays below
    edge = np.array([0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000], np.uint32).view(np.float32)
    assert list(orc.bf16_from_float(edge)) == [0x7F80, 0x7F7F, 0xFF80]


@pytest.mark.parametrize("T,K,H", [(1, 1, 8), (7, 3, 16), (33, 4, 64)])
def test_pack_is_row_scatter(orc, T, K, H):
    rng = np.random.default_rng(T * K)
    x = rng.integers(0, 65536, (T, H)).astype(np.uint16)
    sp = rng.permutation(T * K).astype(np.int32)
    got = orc.pack(x, sp, K)
    ref = np.zeros_like(got)
    ref[sp] = np.repeat(x, K, axis=0)
    assert np.array_equal(got, ref)


def test_pack_skips_negative_rows(orc):
    x = np.arange(3 * 8, dtype=np.uint16).reshape(3, 8)
    sp = np.array([1, -1, -1, 0, 2, -1], np.int32)
    got = orc.pack(x, sp, 2, n_rows=3)
    assert np.array_equal(got, x[[1, 0, 2]])


def test_group_is_row_gather_and_inverse(orc):
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 65536, (50, 24)).astype(np.uint16)
    rp = rng.permutation(50).astype(np.int32)
    got = orc.group(raw, rp)
    assert np.array_equal(got, raw[rp])
    back = orc.group(got, np.argsort(rp).astype(np.int32))
    assert np.array_equal(back, raw)


def test_combine_hand_example(orc):
    # scores 0.75, 0.25 on rows holding 1.0 and 3.0: 0.75 + 0.75 = 1.5 exactly
    y = np.array([[0x3F80] * 8, [0x4040] * 8], np.uint16)  # 1.0, 3.0
    ob, of = orc.combine(y, np.array([0, 1], np.int32), np.array([[0.75, 0.25]], np.float32))
    assert np.all(of == 1.5)
    assert np.all(ob == 0x3FC0)


def test_combine_single_route_is_copy(orc):
    rng = np.random.default_rng(9)
    y = synth.bf16_normal(rng, (40, 32))
    sp = rng.permutation(40).astype(np.int32)
    ob, of = orc.combine(y, sp, np.ones((40, 1), np.float32))
    assert np.array_equal(ob, y[sp])
    assert np.array_equal(of, _f32(y[sp]))


def test_combine_fp64_error_bound_and_rounding(orc):
    rng = np.random.default_rng(21)
    T, K, H = 64, 8, 128
    y = synth.bf16_normal(rng, (T * K + 5, H))
    sp = rng.permutation(T * K + 5)[: T * K].astype(np.int32)
    sp[rng.random(T * K) < 0.15] = -1        # pruned routes contribute nothing
    sc = synth.make_scores(rng, T, K) * np.float32(3.0)
    sc[:, ::3] *= -1                          # signs mixed: cancellation
    ob, of = orc.combine(y, sp, sc)
    terms = np.zeros((T, K, H))
    valid = sp.reshape(T, K) >= 0
    rows = _f32(y[np.maximum(sp, 0)]).astype(np.float64).reshape(T, K, H)
    terms = np.where(valid[:, :, None], sc.astype(np.float64)[:, :, None] * rows, 0.0)
    exact = terms.sum(axis=1)
    bound = 1.01 * (K + 1) * U * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(of.astype(np.float64) - exact) <= bound)
    assert np.array_equal(ob, _bf16_nearest_even(of))


def test_combine_of_identity_experts_returns_x(orc):
    # Dispatch then combine with identity experts and scores summing to one
    # gives back each token's row: the fp32 sum is within a few fp32 ulps of
    # x, far inside half a bf16 ulp, so the rounded output equals x.
    d = synth.make_plan_inputs("tiny")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    send = orc.pack(d["x"], p["send_pos"], K)
    ob, of = orc.combine(send, p["send_pos"], d["scores"][0])
    assert np.array_equal(ob, d["x"])


def _expert_scale(gid):
    return np.float32(1.0 + 0.01 * gid)


def _synthetic_expert(orc):
    def fn(dest, rows, plan):
        cu = plan["inst_cu"][dest]
        n = plan["inst_count"][dest]
        base = plan["inst_gid_base"][dest]
        f = np.empty(rows.shape[0], np.float32)
        for i in range(n):
            f[cu[i]:cu[i + 1]] = _expert_scale(base + i)
        prod = _f32(rows) * f[:, None]          # fp32 product, rounded once
        return orc.bf16_from_float(prod)
    return fn


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_full_chain_over_all_ranks(orc, name):
    # Replays dispatch -> synthetic experts -> combine over every logical
    # rank. Grouped slot t of rank d must hold the row of the route planned
    # into (d, t); the combined output must match the closed form
    # x * sum_k score_k * (1 + 0.01*gid_k) within the bf16 rounding of the
    # expert outputs.
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    C = S * K
    plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    res = orc.chain(d["x_all"], plans, d["scores"], _synthetic_expert(orc))
    dest = plans[0]["route_dest"]
    slot = plans[0]["route_slot"]
    x_route = np.repeat(d["x_all"].reshape(R * S, H), K, axis=0)
    for r in range(R):
        at = np.nonzero(dest == r)[0]
        g = np.empty((C, H), np.uint16)
        g[slot[at]] = x_route[at]
        assert np.array_equal(res[r]["recv_grouped"], g)
    # gid of every route, from the instance tables
    gid_of = np.empty(R * C, np.int64)
    for r in range(R):
        cu = plans[0]["inst_cu"][r]
        for i in range(plans[0]["inst_count"][r]):
            at = np.nonzero((dest == r) & (slot >= cu[i]) & (slot < cu[i + 1]))[0]
            gid_of[at] = plans[0]["inst_gid_base"][r] + i
    for m in range(R):
        sc = d["scores"][m].astype(np.float64)
        f = 1.0 + 0.01 * gid_of[m * C:(m + 1) * C].reshape(S, K)
        xm = _f32(d["x_all"][m]).astype(np.float64)
        approx = xm * (sc * f).sum(axis=1, keepdims=True)
        # y is rounded to bf16 per route: relative error 2^-8 per term
        tol = (2.0 ** -8 + (K + 2) * U) * np.abs(xm) * (np.abs(sc) * f).sum(axis=1, keepdims=True)
        assert np.all(np.abs(res[m]["out_f32"] - approx) <= tol)


def test_ungroup_inverts_group(orc):
    rng = np.random.default_rng(17)
    raw = rng.integers(0, 65536, (40, 16)).astype(np.uint16)
    rp = rng.permutation(40).astype(np.int32)
    g = orc.group(raw, rp)
    assert np.array_equal(orc.ungroup(g, rp), raw)
    ref = np.zeros_like(raw)
    ref[rp] = raw
    assert np.array_equal(orc.ungroup(raw, rp), ref)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_zero_copy_equals_pack_exchange_group(orc, name):
    # Writing every route's row straight to its (destination, slot) gives,
    # for every rank, the buffer that pack -> exchange -> group gives; reading
    # expert outputs in place gives the combine of the returned rows.
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    C = S * K
    plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    res = orc.chain(d["x_all"], plans, d["scores"], _synthetic_expert(orc))
    rd, rs = plans[0]["route_dest"], plans[0]["route_slot"]
    grouped = np.zeros((R, C, H), np.uint16)
    for m in range(R):
        orc.push(d["x_all"][m], rd[m * C:(m + 1) * C], rs[m * C:(m + 1) * C], K, R, C, grouped)
    for r in range(R):
        assert np.array_equal(grouped[r], res[r]["recv_grouped"])
    y_grouped = np.stack([res[r]["y_grouped"] for r in range(R)])
    for m in range(R):
        ob, of = orc.pull_combine(y_grouped, rd[m * C:(m + 1) * C], rs[m * C:(m + 1) * C],
                                  d["scores"][m])
        assert np.array_equal(ob, res[m]["out_bf16"])
        assert np.array_equal(of, res[m]["out_f32"])


# --- the fixed k order and the separate fp32 roundings of the combine -------
# The combine sums in k order from +0, rounding each product and each partial
# sum to fp32 on its own ("MoonEP API完全参考" §3.1 combine; the op doc's
# combine takes the same per-route scales). These vectors give a different
# answer under any other order or rounding: an fp64 accumulator, a reversed
# or pairwise k order, or a fused multiply-add.

def _bf16_rows(vals, H=8):
    """bf16 rows of constant value (each value exact in bf16)."""
    bits = (np.array(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_f32(bits), np.array(vals, np.float32))
    return np.repeat(bits[:, None], H, axis=1)


def test_combine_order_pins_forward_k_sum(orc):
    # rows 1, 2^-24, 2^-24, -1 with unit scores:
    #   in k order: 1 + 2^-24 is a tie that rounds to 1 (even), twice, then
    #               1 - 1 = 0
    #   exact (fp64) 2^-23; reversed order 2^-23; pairwise (1 + 2^-24) +
    #   (2^-24 - 1) = 2^-24
    y = _bf16_rows([1.0, 2.0 ** -24, 2.0 ** -24, -1.0])
    ob, of = orc.combine(y, np.arange(4, dtype=np.int32), np.ones((1, 4), np.float32))
    assert np.all(of == 0.0) and not np.signbit(of).any()
    assert np.all(ob == 0x0000)
    # the first three routes alone: still exactly 1 (a tie kept at 1 twice)
    ob, of = orc.combine(y, np.array([0, 1, 2, -1], np.int32), np.ones((1, 4), np.float32))
    assert np.all(of == 1.0)


def test_combine_pins_separate_product_rounding(orc):
    # route 0: 1 * 1 = 1; route 1: (1 + 2^-23) * (1 + 2^-7)
    #   = 1 + 2^-7 + 2^-23 + 2^-30, rounded alone to 1 + 2^-7 + 2^-23;
    #   1 + that = 2 + 2^-7 + 2^-23, a tie at ulp 2^-22 -> 2 + 2^-7 (even).
    # A fused multiply-add (or fp64) sees the 2^-30 and rounds up to
    # 2 + 2^-7 + 2^-22. bf16 of 2 + 2^-7 is again a tie -> 2.0 (0x4000);
    # of the fused result 2 + 2^-6 (0x4001).
    y = _bf16_rows([1.0, 1.0 + 2.0 ** -7])
    sc = np.array([[1.0, 1.0 + 2.0 ** -23]], np.float32)
    assert sc[0, 1] == np.float32(1.0 + 2.0 ** -23)
    ob, of = orc.combine(y, np.array([0, 1], np.int32), sc)
    assert np.all(of == np.float32(2.0 + 2.0 ** -7))
    assert np.all(ob == 0x4000)


def test_zero_copy_skips_out_of_range_routes(orc):
    # a route whose destination or slot lies outside the R x C grouped
    # buffers is not written by the push and adds nothing to the pull: the
    # result equals the one with that route dropped (pack's -1)
    rng = np.random.default_rng(19)
    T, K, H, R, C = 6, 3, 16, 3, 8
    x = rng.integers(0, 65536, (T, H)).astype(np.uint16)
    rd = rng.integers(0, R, T * K).astype(np.int32)
    rs = rng.integers(0, C, T * K).astype(np.int32)
    bad = np.array([1, 5, 9, 16])
    rd_bad, rs_bad = rd.copy(), rs.copy()
    rd_bad[bad[:2]] = [R, -1]
    rs_bad[bad[2:]] = [C, -1]
    keep = np.ones(T * K, bool)
    keep[bad] = False
    ref = np.zeros((R, C, H), np.uint16)
    for f in np.nonzero(keep)[0]:
        ref[rd[f], rs[f]] = x[f // K]
    assert np.array_equal(orc.push(x, rd_bad, rs_bad, K, R, C), ref)
    # the pull equals the pinned combine over the flattened buffers with the
    # out-of-range routes given position -1
    y = rng.integers(0, 65536, (R, C, H)).astype(np.uint16)
    sc = synth.make_scores(rng, T, K)
    sp = np.where(keep, rd * C + rs, -1).astype(np.int32)
    ob, of = orc.pull_combine(y, rd_bad, rs_bad, sc)
    rb, rf = orc.combine(y.reshape(R * C, H), sp, sc)
    assert np.array_equal(ob, rb) and np.array_equal(of.view(np.uint32), rf.view(np.uint32))
