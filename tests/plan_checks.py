"""Independent checks of a plan: a sequential water-fill simulation and the
properties that characterise the balanced plan.

The balanced plan ("MoonEP" technical overview, architecture section: every
rank processes exactly S*K routed rows, hot experts get temporary copies on
other ranks) is pinned here by two means that share nothing with the oracle's
code:

* ``waterfill``: walks the routes one at a time in (expert, global token, k)
  order, keeping a route on its home rank floor(e*R/E) while that rank has
  taken fewer than C = S*K of its own routes, and otherwise placing it on the
  lowest-numbered under-loaded rank that still has spare room after reserving
  room for its own native routes.
* ``check_plan``: vectorised properties that together determine the plan
  uniquely (bijection onto the R*C slots, keep-first-C per rank, monotone
  spill order, instance layout, send/arrival orders).
"""
from __future__ import annotations

import numpy as np


def waterfill(ids, R, E, S, K):
    ids = [int(v) for v in np.asarray(ids).reshape(-1)]
    C = S * K
    N = R * C
    home = [e * R // E for e in range(E)]
    native = [0] * R
    for e in ids:
        native[home[e]] += 1
    order = sorted(range(N), key=lambda f: (ids[f], f))
    kept = [0] * R
    spilled = [0] * R
    dest = [None] * N
    slot = [None] * N
    for f in order:
        r = home[ids[f]]
        if kept[r] < C:
            dest[f], slot[f] = r, kept[r]
            kept[r] += 1
            continue
        for u in range(R):
            if native[u] < C and native[u] + spilled[u] < C:
                dest[f], slot[f] = u, native[u] + spilled[u]
                spilled[u] += 1
                break
        else:
            raise AssertionError("no room left: loads do not sum to R*C")
    return np.array(dest, np.int32), np.array(slot, np.int32)


def expected_layout(ids, R, E, S, K, route_dest):
    """Per-rank instance list from an assignment: natives ascending (all of
    them, zero-row ones too), then experts homed elsewhere that received rows,
    ascending. Returns lists of (expert, rows)."""
    ids = np.asarray(ids).reshape(-1)
    cnt = np.zeros((R, E), np.int64)
    np.add.at(cnt, (route_dest.astype(np.int64), ids.astype(np.int64)), 1)
    home = (np.arange(E, dtype=np.int64) * R) // E
    lay = []
    for u in range(R):
        nat = [(e, int(cnt[u, e])) for e in range(E) if home[e] == u]
        red = [(e, int(cnt[u, e])) for e in range(E) if home[e] != u and cnt[u, e] > 0]
        lay.append(nat + red)
    return lay


def check_plan(ids, R, E, S, K, m, p):
    """Assert every property of a plan dict (oracle or GPU output)."""
    ids = np.asarray(ids, np.int64).reshape(-1)
    C = S * K
    N = R * C
    dest = p["route_dest"].astype(np.int64)
    slot = p["route_slot"].astype(np.int64)
    home = (np.arange(E, dtype=np.int64) * R) // E

    # histogram and native loads
    cnt = np.bincount(ids, minlength=E)
    assert np.array_equal(p["expert_count"], cnt)
    L = np.bincount(home, weights=cnt, minlength=R).astype(np.int64)
    assert np.array_equal(p["rank_load"], L)

    # bijection onto (dest, slot) in [0,R) x [0,C): every rank gets exactly C
    assert dest.min() >= 0 and dest.max() < R and slot.min() >= 0 and slot.max() < C
    flat = dest * C + slot
    assert np.array_equal(np.sort(flat), np.arange(N))
    assert np.array_equal(np.bincount(dest, minlength=R), np.full(R, C))

    order = np.lexsort((np.arange(N), ids))  # (expert, f) order
    h = home[ids]
    # keep-first-C: routes of home rank r in order, the first min(L,C) stay
    for r in range(R):
        rr = order[h[order] == r]
        k = min(len(rr), C)
        assert np.array_equal(dest[rr[:k]], np.full(k, r))
        assert np.array_equal(slot[rr[:k]], np.arange(k))
        assert np.all(dest[rr[k:]] != r)
    # spill: the excess in global order maps monotonically onto
    # (under-loaded rank ascending, slot ascending) starting at L[u]
    spilled = order[dest[order] != h[order]]
    fill = [(u, s) for u in range(R) if L[u] < C for s in range(L[u], C)]
    assert len(fill) == len(spilled)
    if fill:
        fu = np.array(fill)
        assert np.array_equal(dest[spilled], fu[:, 0])
        assert np.array_equal(slot[spilled], fu[:, 1])

    # instance tables
    lay = expected_layout(ids, R, E, S, K, p["route_dest"])
    gid = 0
    slot_route = np.empty(N, np.int64)
    slot_route[flat] = np.arange(N)
    for u in range(R):
        n = len(lay[u])
        assert p["inst_count"][u] == n
        assert p["inst_gid_base"][u] == gid
        gid += n
        ex = [e for e, _ in lay[u]]
        cu = np.concatenate([[0], np.cumsum([c for _, c in lay[u]])])
        assert np.array_equal(p["inst_expert"][u, :n], ex)
        assert np.all(p["inst_expert"][u, n:] == -1)
        assert np.array_equal(p["inst_cu"][u, : n + 1], cu)
        assert np.all(p["inst_cu"][u, n + 1:] == C)
        # every slot of an instance holds a route of that expert
        for i in range(n):
            rows = slot_route[u * C + cu[i]: u * C + cu[i + 1]]
            assert np.all(ids[rows] == ex[i])
            # rows within an instance are in (global token, k) order
            assert np.all(np.diff(rows) > 0)
    assert p["inst_gid_base"][R] == gid

    # send map of rank m: (dest, slot) order
    mine = np.arange(m * C, (m + 1) * C)
    sp = p["send_pos"].astype(np.int64)
    assert np.array_equal(np.sort(sp), np.arange(C))
    key = dest[mine] * C + slot[mine]
    assert np.all(np.diff(key[np.argsort(sp)]) > 0)
    assert np.array_equal(p["send_count"], np.bincount(dest[mine], minlength=R))

    # arrival order on rank m: (source, slot)
    rp = p["recv_pos"].astype(np.int64)
    assert np.array_equal(np.sort(rp), np.arange(C))
    src = slot_route[m * C: (m + 1) * C] // C
    inv = np.argsort(rp)             # slots in arrival order
    akey = src[inv] * C + inv
    assert np.all(np.diff(akey) > 0)
    assert np.array_equal(p["recv_count"], np.bincount(src, minlength=R))


def maxvio(loads, C):
    """(max load - mean) / mean at rank granularity, mean = C."""
    return float(np.max(loads)) / C - 1.0
