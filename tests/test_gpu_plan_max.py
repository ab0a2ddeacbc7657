"""mep_plan at its largest size, N = R*S*K = 2^30 routes (R=8, E=256,
S=2^24, K=8), with heavily skewed routing.

The oracle's full plan is too slow at this size, so the GPU plan is checked,
with torch's own GPU kernels, against the plan rule written out in
vectorised, block-by-block form ("MoonEP"
technical overview, architecture section: each rank keeps its first C = S*K
routes in (expert, global token, k) order and the excess fills the
under-loaded ranks in ascending order): the exact expert and native-rank
counts, every route's (dest, slot), and this rank's send/arrival maps as
permutations in (dest, slot) and (source, slot) order. Route indices reach
2^30 - 1 here, the bound the kernels' 32-bit offsets rely on. The same
checks run against the oracle's plan at a small size in the CPU suite
(test_oracle_plan.py), so a failure here is the GPU's.
"""
import numpy as np
import pytest

from gpu_util import note, require_gpu

OFFSETS = np.array([0, 1, 3, 7, 15, 31, 63, 127], np.uint8)  # distinct mod 256
BLK = 1 << 26  # routes per checking block (bounds the temporaries)


def skewed_ids(R, S, seed):
    """[R*S*8] uint8 expert ids for E = 256: a zipf-like first expert per
    token, the token's other experts at fixed distinct offsets from it
    (uint8 sums wrap mod 256 = E)."""
    rng = np.random.default_rng(seed)
    w = 1.0 / (np.arange(256) + 1.0)
    cdf = np.cumsum(w) / w.sum()
    # inverse CDF on a 2^16-step grid, indexed by uniform 16-bit draws
    table = np.minimum(np.searchsorted(cdf, (np.arange(1 << 16) + 0.5) / (1 << 16)), 255)
    base = table.astype(np.uint8)[rng.integers(0, 1 << 16, size=R * S, dtype=np.uint16)]
    return (base[:, None] + OFFSETS[None, :]).reshape(-1)


def rule_blocks(ids, R, E, C, blk=BLK):
    """Expert counts, native loads, and every route's (dest, slot) by the
    plan rule, block by block: p(f) is the route's position in (expert, f)
    order (a stable sort of the ids); a route keeps slot
    q = p - (routes of lower home ranks) on its home rank when q < C, else it
    is excess number j = (excess of lower ranks) + q - C, placed on the
    under-loaded rank u whose deficit range holds j, at slot L[u] + j - (the
    deficits below u). ids: an int64 torch tensor on any device."""
    import torch
    dv = ids.device
    N = ids.numel()
    cnt = torch.bincount(ids, minlength=E)
    home = (torch.arange(E, device=dv, dtype=torch.int64) * R) // E
    L = torch.zeros(R, dtype=torch.int64, device=dv).index_add_(0, home, cnt)
    zero = torch.zeros(1, dtype=torch.int64, device=dv)
    rank_begin = torch.cat([zero, torch.cumsum(L, 0)[:-1]])
    U = (L - C).clamp(min=0)
    D = (C - L).clamp(min=0)
    uex = torch.cat([zero, torch.cumsum(U, 0)[:-1]])
    dex = torch.cat([zero, torch.cumsum(D, 0)[:-1]])
    dend = (dex + D).contiguous()
    order = torch.sort(ids, stable=True).indices
    pos = torch.empty_like(order)
    pos[order] = torch.arange(N, device=dv, dtype=torch.int64)
    del order

    def blocks():
        for b0 in range(0, N, blk):
            r = home[ids[b0:b0 + blk]]
            q = pos[b0:b0 + blk] - rank_begin[r]
            j = uex[r] + q - C
            u = torch.searchsorted(dend, j, right=True).clamp_(max=R - 1)
            keep = q < C
            yield b0, torch.where(keep, r, u), torch.where(keep, q, L[u] + j - dex[u])
    return cnt, L, blocks()


def check_plan_at_scale(ids, R, E, S, K, m, p):
    """Assert the plan p (int torch tensors, on the device of ids): every
    route's (dest, slot) by the rule, this rank's send and arrival maps as
    permutations in (dest, slot) and (source, slot) order, and its instances
    covering C slots. Returns the native loads."""
    import torch
    dv = ids.device
    C = S * K
    ids = ids.reshape(-1).to(torch.int64)
    dest = p["route_dest"].reshape(-1)
    slot = p["route_slot"].reshape(-1)
    cnt, L, blocks = rule_blocks(ids, R, E, C)
    assert torch.equal(p["expert_count"].reshape(-1).to(torch.int64), cnt)
    assert torch.equal(p["rank_load"].reshape(-1).to(torch.int64), L)
    for b0, wd, ws in blocks:
        n = wd.numel()
        gd = dest[b0:b0 + n].to(torch.int64)
        gs = slot[b0:b0 + n].to(torch.int64)
        bad = torch.nonzero((gd != wd) | (gs != ws)).reshape(-1)[:4]
        if bad.numel():
            raise AssertionError(f"routes {(bad + b0).tolist()}: got {gd[bad].tolist()}/"
                                 f"{gs[bad].tolist()}, rule {wd[bad].tolist()}/{ws[bad].tolist()}")
        del gd, gs, wd, ws

    # the source rank of each slot on rank m
    mine = torch.nonzero(dest == m).reshape(-1)
    assert mine.numel() == C
    slot_src = torch.full((C,), -1, dtype=torch.int64, device=dv)
    slot_src[slot[mine].to(torch.int64)] = mine // C
    del mine
    assert int(slot_src.min()) >= 0
    ar = torch.arange(C, device=dv, dtype=torch.int64)

    # rank m's send map: a permutation, in (dest, slot) order
    md = dest[m * C:(m + 1) * C].to(torch.int64)
    ms = slot[m * C:(m + 1) * C].to(torch.int64)
    inv = torch.full((C,), -1, dtype=torch.int64, device=dv)
    inv[p["send_pos"].reshape(-1).to(torch.int64)] = ar
    assert int(inv.min()) >= 0
    key = md[inv] * C + ms[inv]
    assert bool(torch.all(key[1:] > key[:-1]))
    assert torch.equal(p["send_count"].reshape(-1).to(torch.int64), torch.bincount(md, minlength=R))
    # rank m's arrival map: a permutation, in (source, slot) order
    inv = torch.full((C,), -1, dtype=torch.int64, device=dv)
    inv[p["recv_pos"].reshape(-1).to(torch.int64)] = ar
    assert int(inv.min()) >= 0
    akey = slot_src[inv] * C + inv
    assert bool(torch.all(akey[1:] > akey[:-1]))
    assert torch.equal(p["recv_count"].reshape(-1).to(torch.int64),
                       torch.bincount(slot_src, minlength=R))
    # rank m's instances cover its C slots
    n = int(p["inst_count"].reshape(-1)[m])
    cu = p["inst_cu"].reshape(R, E + 1)[m].to(torch.int64)
    assert int(cu[0]) == 0 and int(cu[n]) == C and bool(torch.all(cu[1:n + 1] >= cu[:n]))
    return L


@pytest.mark.gpu
def test_plan_at_most_routes():
    torch = require_gpu()
    import combine_balancing_amd as cba
    R, E, S, K, m = 8, 256, 1 << 24, 8, 5
    assert R * S * K == 1 << 30  # the largest plan the library accepts
    ids = skewed_ids(R, S, seed=20261203)
    note(f"plan max size N=2^30 R={R} E={E} S={S} K={K} m={m}")
    d_ids = torch.from_numpy(ids).cuda().to(torch.int32)
    p = cba.plan(d_ids, R, E, S, K, my_rank=m)
    torch.cuda.synchronize()
    # the checks run on the GPU with torch's own kernels (sort, bincount,
    # elementwise), none of the library's
    L = check_plan_at_scale(d_ids, R, E, S, K, m, p)
    assert int(L.max()) > S * K  # the routing spills
    del d_ids, p
    torch.cuda.empty_cache()  # hand the ~40 GiB back before the next test
