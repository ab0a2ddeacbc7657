"""Pins of the oracle's weight-row table under a cap of B prefetch slots.

The pages ("MoonEP" overview, memory contract) describe the group GEMM's
weight tensor [E+B, H, H']: rows 0..E-1 are the experts of all ranks, rows
E..E+B-1 a rank's prefetch slots; B = E/R for training, 3-4 for inference,
with redundant experts beyond the slots served from their home rank. The
oracle's reading is pinned here by properties that fix it on every plan,
checked on the plans of the small workloads and on random routings.
"""
import numpy as np
import pytest

import synth


def _home(e, R, E):
    return (e * R) // E


def _plans(orc):
    for name in ("tiny", "small"):
        d = synth.make_routing(name)
        yield d["R"], d["E"], orc.plan(d["topk_ids"], d["R"], d["E"], d["S"], d["K"], m=0)
    rng = np.random.default_rng(7)
    for R, E, S, K in [(4, 8, 50, 2), (8, 16, 100, 3), (3, 7, 90, 2)]:
        w = np.exp(-2.0 * np.log(np.arange(E) + 1.0))
        g = rng.gumbel(size=(R * S, E)) + np.log(w / w.sum())
        ids = np.argsort(-g, axis=1, kind="stable")[:, :K].astype(np.int32)
        yield R, E, orc.plan(ids, R, E, S, K, m=0)


@pytest.mark.parametrize("B", [0, 1, 3, "E/R", "inf"])
def test_weight_row_properties(orc, B):
    for R, E, p in _plans(orc):
        b = {"E/R": E // R, "inf": E}.get(B, B)
        w = orc.weight_rows(p, R, E, b)
        for u in range(R):
            n = p["inst_count"][u]
            ex = p["inst_expert"][u][:n]
            assert np.all(w[u][n:] == -1)
            nat = np.array([_home(e, R, E) == u for e in ex], bool)
            # natives read their own row
            assert np.array_equal(w[u][:n][nat], ex[nat])
            red = w[u][:n][~nat]
            # the first min(#redundant, B) redundant instances take slots
            # E, E+1, ... in order; the rest read the home rank's row
            m = min(len(red), b)
            assert np.array_equal(red[:m], E + np.arange(m))
            assert np.array_equal(red[m:], ex[~nat][m:])


def test_no_cap_needed_when_balanced(orc):
    # uniform routing over E = R experts with S*K divisible: no copies, so
    # every instance reads its own row whatever B is
    R, E, S, K = 4, 4, 64, 1
    ids = (np.arange(R * S) % E).astype(np.int32).reshape(R * S, 1)
    p = orc.plan(ids, R, E, S, K, m=0)
    w = orc.weight_rows(p, R, E, 0)
    assert np.array_equal(w[:, 0], np.arange(R))
