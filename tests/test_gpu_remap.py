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
