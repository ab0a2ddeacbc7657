"""Pins of the oracle's per-destination dedup maps.

The MoonEP API page names a dedup encoding of sent tokens and nothing more;
the reading (a token is sent once per destination rank and fanned out there
to its grouped slots) is pinned by equivalence with the plan's own, pinned,
dispatch chain, and by counts and orders computed independently with numpy.
"""
import numpy as np
import pytest

import synth


def _exchange(orc, x_all, send_maps, counts, K, R, H):
    """pack each source with its map, then build every rank's arrival
    buffer from the sources' segments (source ascending)."""
    sends = [orc.pack(x_all[m], send_maps[m], K, n_rows=int(counts[m].sum()))
             for m in range(R)]
    off = [np.concatenate([[0], np.cumsum(counts[m])]) for m in range(R)]
    return [np.concatenate([sends[src][off[src][d]:off[src][d + 1]] for src in range(R)])
            .reshape(-1, H) for d in range(R)]


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_dedup_chain_equals_plain_chain(orc, name):
    d = synth.make_plan_inputs(name)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    plans = [orc.plan(d["topk_ids"], R, E, S, K, m=m) for m in range(R)]
    dd = [orc.plan_dedup(plans[0], R, S, K, m) for m in range(R)]
    # plain chain
    raw = _exchange(orc, d["x_all"], [p["send_pos"] for p in plans],
                    np.array([p["send_count"] for p in plans]), K, R, H)
    # dedup chain
    draw = _exchange(orc, d["x_all"], [q["dpack_pos"] for q in dd],
                     np.array([q["dsend_count"] for q in dd]), K, R, H)
    for r in range(R):
        assert draw[r].shape[0] == dd[r]["drecv_count"].sum()
        assert np.array_equal(orc.group(draw[r], dd[r]["drecv_pos"]),
                              orc.group(raw[r], plans[r]["recv_pos"]))


def test_counts_and_orders(orc):
    d = synth.make_routing("small")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    dest = p["route_dest"].reshape(R, S, K)
    for m in (0, R - 1):
        q = orc.plan_dedup(p, R, S, K, m)
        # distinct (token, dest) pairs of source m, by numpy sets
        has = np.zeros((S, R), bool)
        for k in range(K):
            has[np.arange(S), dest[m, :, k]] = True
        assert np.array_equal(q["dsend_count"], has.sum(axis=0))
        # rows: a bijection onto [0, #pairs), in (dest, token) order
        rows = q["dpack_pos"].reshape(S, K)
        keep = rows >= 0
        assert keep.sum() == has.sum()
        pairs = sorted((dest[m, t, k], t, rows[t, k]) for t in range(S) for k in range(K)
                       if keep[t, k])
        assert [r for _, _, r in pairs] == list(range(len(pairs)))
        # the first route of each (token, dest) carries the row
        for t in range(S):
            seen = set()
            for k in range(K):
                assert keep[t, k] == (dest[m, t, k] not in seen)
                seen.add(dest[m, t, k])
        # tokens arriving at m per source
        reach = (dest == m).any(axis=2)
        assert np.array_equal(q["drecv_count"], reach.sum(axis=1))


def test_dedup_saves_rows_on_headline_routing(orc):
    # with K = 8 routes over R = 8 ranks a token reaches about 5.3 distinct
    # ranks, so the dedup send buffer holds roughly two thirds of C rows
    d = synth.make_routing("dsv3")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    q = orc.plan_dedup(p, R, S, K, 0)
    frac = q["dsend_count"].sum() / (S * K)
    assert 0.5 < frac < 0.8
