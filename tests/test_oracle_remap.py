"""Pins of the oracle's EPLB remap, pruning and send map.

Source: "aclnnMoeUpdateExpert" op doc, section "功能说明" (function
description): load balancing maps each (token, k) logical expert to one of the
instances listed in its eplb_table row (balance_mode 0 by rank, 1 by token);
pruning drops a route whose scale is below the token's sum of
scale x threshold, and drops every route of an inactive token.
"""
import numpy as np
import pytest

import golden_io


def test_pages_identity_example(orc):
    g = golden_io.read("remap_identity_ep2.txt")
    table = np.array(g["eplb_table"], np.int32).reshape(-1, g["F"])
    ids = np.array(g["expert_ids"], np.int32).reshape(g["BS"], g["K"])
    for rank in g["local_rank_ids"]:
        out = orc.remap_prune(ids, table, g["world_size"], g["place_per_rank"],
                              rank, g["balance_mode"])
        assert out["balanced_ids"].reshape(-1).tolist() == g["balanced_ids"]
        # no scales and no threshold: nothing is pruned
        assert np.all(out["balanced_mask"] == 1)


def test_modes_on_a_three_instance_row(orc):
    # Row of expert 0: count 3, instances 10, 20, 30; world size 8.
    # Mode 0: column = rank / ceil(8/3) + 1 = rank // 3 + 1 -> ranks 0-2 take
    # 10, ranks 3-5 take 20, ranks 6-7 take 30.
    # Mode 1: column = t mod 3 + 1 -> tokens 0,1,2,3 take 10,20,30,10.
    table = np.array([[3, 10, 20, 30, 0], [1, 7, 0, 0, 0]], np.int32)
    ids = np.array([[0, 1], [0, 1], [0, 1], [0, 1]], np.int32)
    exp0 = {0: 10, 1: 10, 2: 10, 3: 20, 4: 20, 5: 20, 6: 30, 7: 30}
    for rank, inst in exp0.items():
        out = orc.remap_prune(ids, table, 8, 4, rank, 0)
        assert out["balanced_ids"][:, 0].tolist() == [inst] * 4
        assert out["balanced_ids"][:, 1].tolist() == [7] * 4   # count 1
    out = orc.remap_prune(ids, table, 8, 4, 5, 1)
    assert out["balanced_ids"][:, 0].tolist() == [10, 20, 30, 10]
    assert out["balanced_ids"][:, 1].tolist() == [7] * 4


def test_mode0_columns_stay_within_count(orc):
    # For every count c in [1, ws] and rank in [0, ws), the chosen column is
    # in [1, c]: rank // ceil(ws/c) <= (ws-1) // ceil(ws/c) < c.
    ws = 13
    E = ws
    F = ws + 1
    table = np.zeros((E, F), np.int32)
    for e in range(E):
        c = e + 1
        table[e, 0] = c
        table[e, 1:] = 1000 + np.arange(F - 1)          # column j -> 1000+j-1
    ids = np.arange(E, dtype=np.int32).reshape(E, 1)
    for rank in range(ws):
        out = orc.remap_prune(ids, table, ws, 2000, rank, 0, want_send=False)
        col = out["balanced_ids"][:, 0] - 1000 + 1
        counts = table[:, 0]
        assert np.all(col >= 1) and np.all(col <= counts)
        # every rank in a group of ceil(ws/c) shares one column
        assert np.array_equal(col, [1 if c == 1 else rank // -(-ws // c) + 1 for c in counts])


def _bf16(v):
    return (np.array(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_prune_examples(orc):
    table = np.array([[1, 0], [1, 1], [1, 2]], np.int32)
    ids = np.array([[0, 1], [1, 2], [2, 0]], np.int32)
    thr = np.array([0.5, 0.5], np.float32)
    # token 0: scales 0.75, 0.25 -> sum 0.375+0.125 = 0.5 -> keep 0.75, drop 0.25
    # token 1: scales 0.5, 0.5 -> sum 0.5 -> both equal the sum -> both kept
    # token 2: inactive -> both dropped
    scales = _bf16([[0.75, 0.25], [0.5, 0.5], [0.75, 0.25]])
    active = np.array([1, 1, 0], np.uint8)
    out = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=scales,
                          pruning_threshold=thr, active_mask=active)
    assert out["balanced_mask"].tolist() == [[1, 0], [1, 1], [0, 0]]
    # send map: kept routes in (card, instance, t, k) order, -1 when pruned
    # kept: (0,0)->inst 0, (1,0)->inst 1, (1,1)->inst 2
    assert out["send_pos"].tolist() == [0, -1, 1, 2, -1, -1]
    assert out["send_count"].tolist() == [1, 1, 1]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_prune_dtypes_agree_on_exact_values(orc, dtype):
    # Values exactly representable in all three formats give the same mask.
    table = np.array([[1, 0]] * 4, np.int32)
    ids = np.array([[0, 1, 2, 3]] * 2, np.int32)
    v = np.array([[0.5, 0.25, 0.125, 0.125], [0.375, 0.375, 0.125, 0.125]], np.float32)
    thr = np.array([0.25, 0.25, 0.25, 0.25], np.float32)
    if dtype == "fp32":
        sc = v
    elif dtype == "bf16":
        sc = _bf16(v)
    else:
        sc = v.astype(np.float16).view(np.uint16)
    out = orc.remap_prune(ids, table, 1, 4, 0, 0, expert_scales=sc,
                          scale_dtype=dtype, pruning_threshold=thr)
    # sums: 0.25 and 0.25; kept where scale >= 0.25
    assert out["balanced_mask"].tolist() == [[1, 1, 0, 0], [1, 1, 0, 0]]


def test_fp16_widening_matches_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.float_from_fp16(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_eplb_workload_mask_is_prefix_and_matches_fp64(orc):
    import synth
    d = synth.make_eplb_inputs(with_x=False)
    for mode, rank in [(0, 0), (0, 191), (1, 0)]:
        out = orc.remap_prune(d["expert_ids"], d["eplb_table"], d["world_size"],
                              d["place_per_rank"], rank, mode,
                              expert_scales=d["expert_scales"],
                              pruning_threshold=d["pruning_threshold"],
                              active_mask=d["active_mask"])
        mask = out["balanced_mask"].astype(bool)
        # scales are descending per token and active tokens come first, so
        # each token keeps a prefix of its k and inactive tokens keep nothing
        assert np.all(mask[:, 1:] <= mask[:, :-1])
        assert not mask[~d["active_mask"].astype(bool)].any()
        assert mask[d["active_mask"].astype(bool), 0].all()
        # decisions far from the boundary agree with an fp64 evaluation
        s = (d["expert_scales"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ssum = (s * d["pruning_threshold"].astype(np.float64)).sum(axis=1, keepdims=True)
        far = np.abs(s - ssum) > 1e-6 * ssum
        ref = (s >= ssum) & d["active_mask"].astype(bool)[:, None]
        assert np.array_equal(mask[far], ref[far])
        # remap: each id maps to one of the instances its row lists
        tab = d["eplb_table"]
        bal = out["balanced_ids"]
        cnt = tab[d["expert_ids"], 0]
        cols = [[np.nonzero(tab[e, 1:] == b)[0] for e, b in zip(er, br)]
                for er, br in zip(d["expert_ids"], bal)]
        for row, crow in zip(cnt, cols):
            for c, idx in zip(row, crow):
                assert len(idx) == 1 and idx[0] < c
        # send map: permutation of the kept routes, ordered by instance
        sp = out["send_pos"]
        kept = sp >= 0
        assert np.array_equal(kept, mask.reshape(-1))
        assert np.array_equal(np.sort(sp[kept]), np.arange(kept.sum()))
        inst = bal.reshape(-1)[kept]
        by_row = np.argsort(sp[kept])
        key = inst[by_row].astype(np.int64) * 10**6 + np.nonzero(kept)[0][by_row]
        assert np.all(np.diff(key) > 0)
        card = bal.reshape(-1)[kept] // d["place_per_rank"]
        assert np.array_equal(out["send_count"],
                              np.bincount(card, minlength=d["world_size"]))


def test_rejects_unpaired_optionals(orc):
    table = np.array([[1, 0]], np.int32)
    ids = np.zeros((1, 1), np.int32)
    with pytest.raises(orc.OracleError):
        orc.remap_prune(ids, table, 2, 1, 0, 0, expert_scales=_bf16([[1.0]]))
    with pytest.raises(orc.OracleError):
        orc.remap_prune(ids, table, 2, 1, 0, 0, active_mask=np.ones(1, np.uint8))
    with pytest.raises(orc.OracleError):
        orc.remap_prune(ids, table, 2, 1, 0, 2)


# --- the prune threshold sum: fp32, k order, products rounded alone ---------
# "aclnnMoeUpdateExpert" 功能说明: a route is pruned when its scale is below
# the token's sum of scale x threshold. The reading (R-h) fixes that sum as
# fp32, added in k order from +0 with each product rounded on its own. These
# tokens flip their mask under an fp64 (or reversed-order) sum, or under a
# fused multiply-add.

def test_prune_sum_is_sequential_fp32(orc):
    # unit scales, thresholds 1, 2^-24, 2^-24: products 1, 2^-24, 2^-24.
    #   k order: 1 + 2^-24 is a tie -> 1 (even), twice: sum 1, so every
    #            scale (1) equals the sum and is kept.
    #   fp64 or reversed order: 1 + 2^-23 > 1, every route pruned.
    table = np.array([[1, 0], [1, 1], [1, 2]], np.int32)
    ids = np.array([[0, 1, 2]], np.int32)
    thr = np.array([1.0, 2.0 ** -24, 2.0 ** -24], np.float32)
    out = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=_bf16([[1.0, 1.0, 1.0]]),
                          pruning_threshold=thr)
    assert out["balanced_mask"].tolist() == [[1, 1, 1]]
    # the thresholds reversed: 2^-24 + 2^-24 = 2^-23 first, then 1 + 2^-23
    # is exact, so the sum exceeds 1 and all three routes are pruned
    out = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=_bf16([[1.0, 1.0, 1.0]]),
                          pruning_threshold=thr[::-1].copy())
    assert out["balanced_mask"].tolist() == [[0, 0, 0]]


def test_prune_products_rounded_before_the_add(orc):
    # fp32 scales 1, 1 + 2^-7, 2 + 2^-7 with thresholds 1, 1 + 2^-23, 0:
    #   products 1, fl(1 + 2^-7 + 2^-23 + 2^-30) = 1 + 2^-7 + 2^-23, 0;
    #   1 + (1 + 2^-7 + 2^-23) = 2 + 2^-7 + 2^-23 is a tie at ulp 2^-22 and
    #   rounds to 2 + 2^-7 (even). The third scale equals the sum: kept.
    #   A fused multiply-add (or fp64) keeps the 2^-30 and the sum rounds up
    #   to 2 + 2^-7 + 2^-22: the third route would be pruned.
    table = np.array([[1, 0], [1, 1], [1, 2]], np.int32)
    ids = np.array([[0, 1, 2]], np.int32)
    sc = np.array([[1.0, 1.0 + 2.0 ** -7, 2.0 + 2.0 ** -7]], np.float32)
    thr = np.array([1.0, 1.0 + 2.0 ** -23, 0.0], np.float32)
    out = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=sc, scale_dtype="fp32",
                          pruning_threshold=thr)
    assert out["balanced_mask"].tolist() == [[0, 0, 1]]


def test_mode0_groups_partition_the_ranks(orc):
    # Reading R-d as a structure, not a formula: over ranks 0..ws-1 the mode-0
    # column of a count-c row starts at 1, never decreases, rises by one
    # between groups, and every group of equal columns but the last holds
    # ceil(ws/c) ranks (the last holds the rest). Checked for every
    # world size up to 40 and every count up to 12 that fits it.
    for ws in range(1, 41):
        counts = [c for c in range(1, 13) if c <= ws]
        F = max(counts) + 1
        table = np.zeros((len(counts), F), np.int32)
        for i, c in enumerate(counts):
            table[i, 0] = c
            table[i, 1:] = 1000 + np.arange(F - 1)
        ids = np.arange(len(counts), dtype=np.int32).reshape(-1, 1)
        cols = np.stack([orc.remap_prune(ids, table, ws, 2000, r, 0, want_send=False)
                         ["balanced_ids"][:, 0] - 999 for r in range(ws)])   # [rank, row]
        for i, c in enumerate(counts):
            seq = cols[:, i]
            assert seq[0] == 1 and np.all(np.diff(seq) >= 0) and np.all(np.diff(seq) <= 1)
            assert seq.max() <= c
            if c == 1:
                assert np.all(seq == 1)
                continue
            size = -(-ws // c)
            runs = np.diff(np.flatnonzero(np.diff(np.r_[0, seq, seq[-1] + 1])))
            assert np.all(runs[:-1] == size) and 1 <= runs[-1] <= size, (ws, c, seq)


def test_mode1_cycles_over_tokens(orc):
    # Reading R-b/R-c as a structure: in mode 1, over consecutive tokens the
    # column of a count-c row starts at 1 and advances by one, wrapping from
    # c back to 1. Every token routes to every row (K = E = 8, counts 1 to 8),
    # in a different order per token.
    counts = list(range(1, 9))
    F = 9
    table = np.zeros((len(counts), F), np.int32)
    for i, c in enumerate(counts):
        table[i, 0] = c
        table[i, 1:] = 1000 + np.arange(F - 1)
    BS, K = 50, len(counts)
    rng = np.random.default_rng(3)
    ids = np.stack([rng.permutation(K) for _ in range(BS)]).astype(np.int32)
    out = orc.remap_prune(ids, table, 64, 8, 0, 1, want_send=False)
    col = out["balanced_ids"] - 999
    for e, c in enumerate(counts):
        seq = col[ids == e]            # one per token, in token order
        assert len(seq) == BS and seq[0] == 1
        assert np.all(seq[1:] == np.where(seq[:-1] == c, 1, seq[:-1] + 1)), (c, seq)
