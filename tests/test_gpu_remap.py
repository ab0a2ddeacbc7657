"""GPU parity of mep_remap_prune against the oracle (bit-exact)."""
import numpy as np
import pytest

import golden_io
import synth
from gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu


def _gpu(ids, table, ws, ppr, rank, mode, scales=None, sdt="bf16", thr=None, active=None,
         want_send=True):
    torch = require_gpu()
    import combine_balancing_amd as cba
    out = cba.remap_prune(dev(ids), dev(table), ws, ppr, rank, mode,
                          expert_scales=None if scales is None else dev(scales),
                          pruning_threshold=None if thr is None else dev(thr),
                          active_mask=None if active is None else dev(active),
                          scale_dtype=sdt, want_send=want_send)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _cmp(ref, got, ctx):
    for k in ref:
        assert np.array_equal(np.asarray(ref[k]).reshape(-1), np.asarray(got[k]).reshape(-1)), \
            f"{ctx}: {k}"


@pytest.mark.parametrize("mode,rank", [(0, 0), (0, 1), (0, 191), (0, 383), (1, 0)])
def test_eplb_workload(orc, mode, rank):
    require_gpu()
    d = synth.make_eplb_inputs(with_x=False)
    note(f"remap eplb mode={mode} rank={rank}")
    args = (d["expert_ids"], d["eplb_table"], d["world_size"], d["place_per_rank"], rank, mode)
    kw = dict(scales=d["expert_scales"], thr=d["pruning_threshold"], active=d["active_mask"])
    got = _gpu(*args, **kw)
    ref = orc.remap_prune(*args, expert_scales=d["expert_scales"],
                          pruning_threshold=d["pruning_threshold"], active_mask=d["active_mask"])
    _cmp(ref, got, f"mode={mode} rank={rank}")


def test_pages_identity_example(orc):
    require_gpu()
    g = golden_io.read("remap_identity_ep2.txt")
    table = np.array(g["eplb_table"], np.int32).reshape(-1, g["F"])
    ids = np.array(g["expert_ids"], np.int32).reshape(g["BS"], g["K"])
    for rank in g["local_rank_ids"]:
        note(f"remap identity example rank={rank}")
        got = _gpu(ids, table, g["world_size"], g["place_per_rank"], rank, g["balance_mode"])
        assert got["balanced_ids"].reshape(-1).tolist() == g["balanced_ids"]
        assert np.all(got["balanced_mask"] == 1)
        ref = orc.remap_prune(ids, table, g["world_size"], g["place_per_rank"], rank,
                              g["balance_mode"])
        _cmp(ref, got, "identity")


@pytest.mark.parametrize("sdt", ["fp32", "bf16", "fp16"])
def test_scale_dtypes_and_optionals(orc, sdt):
    require_gpu()
    rng = np.random.default_rng({"fp32": 1, "bf16": 2, "fp16": 3}[sdt])
    BS, K, E, ws, ppr = 300, 6, 40, 17, 3
    F = 7
    table = np.zeros((E, F), np.int32)
    table[:, 0] = rng.integers(1, F, E)
    for e in range(E):
        table[e, 1:] = rng.choice(ws * ppr, F - 1, replace=False)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(BS)]).astype(np.int32)
    v = -np.sort(-rng.random((BS, K)).astype(np.float32), axis=1)
    v /= v.sum(axis=1, keepdims=True)
    if sdt == "fp32":
        sc = v.astype(np.float32)
    elif sdt == "bf16":
        sc = synth.bf16_from_f32_trunc(v)
    else:
        sc = v.astype(np.float16).view(np.uint16)
    thr = rng.uniform(0, 0.4, K).astype(np.float32)
    active = (np.arange(BS) < 250).astype(np.uint8)
    for mode, rank in [(0, 0), (0, 16), (1, 5)]:
        note(f"remap {sdt} mode={mode} rank={rank}")
        ref = orc.remap_prune(ids, table, ws, ppr, rank, mode, expert_scales=sc,
                              scale_dtype=sdt, pruning_threshold=thr, active_mask=active)
        got = _gpu(ids, table, ws, ppr, rank, mode, scales=sc, sdt=sdt, thr=thr, active=active)
        _cmp(ref, got, f"{sdt} mode={mode}")
        # scales and threshold without an active mask
        ref = orc.remap_prune(ids, table, ws, ppr, rank, mode, expert_scales=sc,
                              scale_dtype=sdt, pruning_threshold=thr)
        got = _gpu(ids, table, ws, ppr, rank, mode, scales=sc, sdt=sdt, thr=thr)
        _cmp(ref, got, f"{sdt} mode={mode} no active")
    # nothing optional, no send map
    ref = orc.remap_prune(ids, table, ws, ppr, 3, 0, want_send=False)
    got = _gpu(ids, table, ws, ppr, 3, 0, want_send=False)
    _cmp(ref, got, "bare")


def test_largest_sizes(orc):
    require_gpu()
    rng = np.random.default_rng(77)
    BS, K, E, ws, ppr, F = 512, 16, 1024, 1024, 1, 17
    table = np.zeros((E, F), np.int32)
    table[:, 0] = rng.integers(1, F, E)
    for e in range(E):
        table[e, 1:] = rng.choice(ws * ppr, F - 1, replace=False)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(BS)]).astype(np.int32)
    sc = synth.bf16_from_f32_trunc(-np.sort(-rng.random((BS, K)).astype(np.float32), axis=1) / K)
    thr = rng.uniform(0, 0.2, K).astype(np.float32)
    for mode in (0, 1):
        note(f"remap largest mode={mode}")
        ref = orc.remap_prune(ids, table, ws, ppr, 1023, mode, expert_scales=sc,
                              pruning_threshold=thr)
        got = _gpu(ids, table, ws, ppr, 1023, mode, scales=sc, thr=thr)
        _cmp(ref, got, f"largest mode={mode}")


def test_rejects_unpaired_optionals():
    torch = require_gpu()
    import combine_balancing_amd as cba
    from combine_balancing_amd import _binding as B
    ids = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    table = torch.tensor([[1, 0], [1, 1]], dtype=torch.int32, device="cuda")
    sc = torch.ones(2, 2, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MepError):
        cba.remap_prune(ids, table, 2, 1, 0, 0, expert_scales=sc)
    with pytest.raises(B.MepError):
        cba.remap_prune(ids, table, 2, 1, 2, 0)


def test_prune_order_vectors(orc):
    # tokens whose mask flips under an fp64 or reversed-order threshold sum
    # or a fused multiply-add: the kernel takes the oracle's decisions
    require_gpu()
    table = np.array([[1, 0], [1, 1], [1, 2]], np.int32)
    ids = np.array([[0, 1, 2], [0, 1, 2]], np.int32)
    one = 0x3F80
    thr = np.array([1.0, 2.0 ** -24, 2.0 ** -24], np.float32)
    for t, want in ((thr, 1), (thr[::-1].copy(), 0)):
        note(f"prune order vector thr={t.tolist()}")
        sc = np.full((2, 3), one, np.uint16)
        got = _gpu(ids, table, 3, 1, 0, 0, scales=sc, thr=t)
        ref = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=sc, pruning_threshold=t)
        _cmp(ref, got, "prune order")
        assert np.all(got["balanced_mask"] == want)
    sc = np.array([[1.0, 1.0 + 2.0 ** -7, 2.0 + 2.0 ** -7]] * 2, np.float32)
    thr = np.array([1.0, 1.0 + 2.0 ** -23, 0.0], np.float32)
    note("prune product-rounding vector")
    got = _gpu(ids, table, 3, 1, 0, 0, scales=sc, sdt="fp32", thr=thr)
    ref = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=sc, scale_dtype="fp32",
                          pruning_threshold=thr)
    _cmp(ref, got, "prune product rounding")
    assert got["balanced_mask"].tolist() == [[0, 0, 1], [0, 0, 1]]


def test_prune_subnormal_scales(orc):
    # bf16 scales down in the fp32 subnormal range: products and sums that
    # are subnormal decide masks (a kernel that flushed them to zero would
    # keep token 0's first route: its scale would then equal the sum)
    require_gpu()
    table = np.array([[1, 0], [1, 1], [1, 2]], np.int32)
    ids = np.array([[0, 1, 2]] * 4, np.int32)
    sc = np.array([[0x0080, 0x0040, 0x0001],    # 2^-126, 2^-127, 2^-133
                   [0x0040, 0x0020, 0x0010],
                   [0x0100, 0x0003, 0x8001],
                   [0x3F80, 0x0001, 0x0001]], np.uint16)
    thr = np.array([1.0, 1.0, 0.75], np.float32)
    note("prune with subnormal bf16 scales")
    got = _gpu(ids, table, 3, 1, 0, 0, scales=sc, thr=thr)
    ref = orc.remap_prune(ids, table, 3, 1, 0, 0, expert_scales=sc, pruning_threshold=thr)
    _cmp(ref, got, "subnormal scales")
    assert got["balanced_mask"][0].tolist() == [0, 0, 0]


def test_random_shapes(orc):
    """Thirty seeded shapes: BS, K, E, F, world size and instances per card
    drawn over their limits, both modes, all three scale types, with and
    without the active mask and the send map."""
    require_gpu()
    rng = np.random.default_rng(20261205)
    for case in range(30):
        ws = int(rng.integers(1, 1025))
        ppr = int(rng.integers(1, max(2, 1024 // ws + 1)))
        ppr = min(ppr, 1024 // ws)
        E = int(rng.integers(1, 1025))
        K = int(rng.integers(1, min(E, 16) + 1))
        BS = int(rng.integers(1, 513))
        F = int(rng.integers(2, min(ws + 1, 17) + 1))
        n_inst = ws * ppr
        table = np.zeros((E, F), np.int32)
        table[:, 0] = rng.integers(1, F, E)
        for e in range(E):
            table[e, 1:] = rng.choice(n_inst, F - 1, replace=n_inst < F - 1)
        ids = np.argsort(rng.random((BS, E)), axis=1)[:, :K].astype(np.int32)
        mode = int(rng.integers(0, 2))
        rank = int(rng.integers(0, ws))
        sdt = str(rng.choice(["fp32", "bf16", "fp16"]))
        v = -np.sort(-rng.random((BS, K)).astype(np.float32), axis=1)
        v /= v.sum(axis=1, keepdims=True)
        sc = {"fp32": v, "bf16": synth.bf16_from_f32_trunc(v),
              "fp16": v.astype(np.float16).view(np.uint16)}[sdt]
        thr = rng.uniform(0, 0.3, K).astype(np.float32)
        active = (rng.random(BS) < 0.9).astype(np.uint8) if rng.random() < 0.5 else None
        want_send = bool(rng.random() < 0.8)
        prune = bool(rng.random() < 0.8)
        note(f"remap random case {case}: BS={BS} K={K} E={E} F={F} ws={ws} ppr={ppr} "
             f"mode={mode} rank={rank} {sdt} prune={prune} active={active is not None}")
        kw = dict(expert_scales=sc, scale_dtype=sdt, pruning_threshold=thr,
                  active_mask=active) if prune else {}
        ref = orc.remap_prune(ids, table, ws, ppr, rank, mode, want_send=want_send, **kw)
        got = _gpu(ids, table, ws, ppr, rank, mode, scales=sc if prune else None, sdt=sdt,
                   thr=thr if prune else None, active=active if prune else None,
                   want_send=want_send)
        _cmp(ref, got, f"case {case}")


# The kernel is compiled for 1, 2, 4 or 8 batches of 64 entries per wave
# (BS*K up to 1024, 2048, 4096 and 8192 over its 16 waves), each with the
# table staged in LDS (E*F <= 9216) or read from global memory. Every
# variant runs at the top of its range and on a ragged size inside it.
VARIANT_CASES = [
    # (BS, K, E, F): staged tables (E*F <= 9216), then tables in global memory
    (64, 16, 600, 9), (7, 5, 600, 9), (128, 16, 700, 13), (65, 16, 700, 13),
    (256, 16, 1000, 9), (129, 16, 1000, 9), (512, 16, 512, 17), (300, 15, 512, 17),
    (64, 16, 1024, 10), (7, 5, 1024, 10), (128, 16, 1000, 12), (65, 16, 1000, 12),
    (256, 16, 1024, 17), (129, 16, 1024, 17), (512, 16, 1024, 11), (300, 15, 1024, 11),
]


@pytest.mark.parametrize("BS,K,E,F", VARIANT_CASES)
def test_batch_and_table_variants(orc, BS, K, E, F):
    require_gpu()
    rng = np.random.default_rng(BS * 131 + K * 17 + E + F)
    ws, ppr = 300, 3
    table = np.zeros((E, F), np.int32)
    table[:, 0] = rng.integers(1, F, E)
    for e in range(E):
        table[e, 1:] = rng.choice(ws * ppr, F - 1, replace=False)
    ids = np.argsort(rng.random((BS, E)), axis=1)[:, :K].astype(np.int32)
    v = -np.sort(-rng.random((BS, K)).astype(np.float32), axis=1)
    sc = synth.bf16_from_f32_trunc(v / v.sum(axis=1, keepdims=True))
    thr = rng.uniform(0, 0.3, K).astype(np.float32)
    active = (rng.random(BS) < 0.9).astype(np.uint8)
    for mode in (0, 1):
        note(f"remap variant BS={BS} K={K} E={E} F={F} mode={mode}")
        ref = orc.remap_prune(ids, table, ws, ppr, 7, mode, expert_scales=sc,
                              pruning_threshold=thr, active_mask=active)
        got = _gpu(ids, table, ws, ppr, 7, mode, scales=sc, thr=thr, active=active)
        _cmp(ref, got, f"BS={BS} K={K} E={E} F={F} mode={mode}")
