"""GPU parity of mep_combine_add_rmsnorm against the oracle.

x_out is compared bit for bit (the same fp32 operations in the same order as
the oracle). rstd and y depend on the sum of squares, which the kernel
forms in fp64 as the oracle does: each square of an fp32 value is exact in
fp64 and the sum's relative error is of order 1e-15, whatever the row's
magnitude. rstd is then rounded to fp32 (2^-24 relative), after an eps
that the kernel takes as fp32 (at most 2^-25 relative in rstd), so rstd is
within 2^-23 relative. y = (x * rstd) * gamma takes two more fp32 roundings
and the bf16 rounding (at most 2^-8 of |y|), so |y - y_exact| <=
|y_exact| * (2^-8 + 2^-21) + 1e-30.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

RSTD_TOL = 2.0 ** -23
Y_TOL = 2.0 ** -8 + 2.0 ** -21


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _inputs(T, K, H, n_y, seed, prune=0.15, scale=1.0):
    rng = np.random.default_rng(seed)
    y = synth.bf16_normal(rng, (max(n_y, 1), H))[:n_y]
    sp = rng.integers(0, max(n_y, 1), T * K).astype(np.int32) if n_y else np.full(T * K, -1, np.int32)
    sp[rng.random(T * K) < prune] = -1
    sc = synth.make_scores(rng, T, K)
    res = synth.bf16_normal(rng, (T, H))
    if scale != 1.0:
        res = (( _f32(res) * np.float32(scale)).view(np.uint32) >> 16).astype(np.uint16)
    g = synth.bf16_normal(rng, (H,))
    return y, sp, sc, res, g


def _check(orc, y, sp, sc, res, g, eps, rows=None, n_y=None):
    torch = require_gpu()
    import combine_balancing_amd as cba
    T, K = sc.shape
    H = res.shape[1]
    yd = dev(y) if y.shape[0] else None
    yo, xo, rs = cba.combine_add_rmsnorm(yd, dev(sp), dev(sc), dev(res), dev(g), eps=eps)
    torch.cuda.synchronize()
    yo, xo, rs = host(yo), host(xo), host(rs)
    if rows is None:
        rows = np.arange(T)
    ref = orc.combine_add_rmsnorm(y if y.shape[0] else np.zeros((1, H), np.uint16),
                                  sp.reshape(T, K)[rows], sc[rows], res[rows], g, eps,
                                  n_y=y.shape[0] if n_y is None else n_y)
    assert np.array_equal(xo[rows], ref["x_out"])
    rel = np.abs(rs[rows].astype(np.float64) - ref["rstd"]) / ref["rstd"]
    assert rel.max() <= RSTD_TOL, rel.max()
    yg = _f32(yo[rows]).astype(np.float64)
    err = np.abs(yg - ref["y"])
    bound = np.abs(ref["y"]) * Y_TOL + 1e-30
    assert np.all(err <= bound), (err / np.maximum(np.abs(ref["y"]), 1e-30)).max()


def _scaled(bits, f):
    """bf16 patterns times a power of two (exact while in range)."""
    return ((_f32(bits) * np.float32(f)).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("f", [2.0 ** -70, 2.0 ** 70])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_fused_norm_tiny_and_huge_rows(orc, f, eps):
    # rows whose squares fall below fp32's normal range (2^-70: x^2 near
    # 2^-146) or above it (2^70: x^2 near 2^140) are normalised as any
    # other, the squares being summed in fp64
    note(f"fused norm rows scaled by 2^{int(np.log2(f))} eps={eps}")
    T, K, H = 24, 8, 1024
    y, sp, sc, res, g = _inputs(T, K, H, 120, 4242)
    _check(orc, _scaled(y, f), sp, sc, _scaled(res, f), g, eps)


CASES = [
    # T, K, H, n_y: one row; short rows sharing a work-group; ragged vectors
    # per thread; every compiled K and the generic path; the H limit
    (1, 1, 8, 4), (5, 3, 24, 20), (64, 8, 128, 600), (77, 2, 1032, 150), (33, 4, 2048, 140),
    (19, 6, 5120, 120), (40, 8, 7168, 330), (9, 16, 4096, 150), (7, 5, 16384, 40),
    (300, 8, 7168, 2400), (130, 1, 256, 130),
]


@pytest.mark.parametrize("T,K,H,n_y", CASES)
def test_fused_norm_shapes(orc, T, K, H, n_y):
    note(f"combine_add_rmsnorm T={T} K={K} H={H}")
    y, sp, sc, res, g = _inputs(T, K, H, n_y, seed=T * 131 + K * 7 + H)
    _check(orc, y, sp, sc, res, g, 1e-6)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_fused_norm_eps_and_scale(orc, eps):
    # small and large magnitudes: eps matters for the small rows
    note(f"combine_add_rmsnorm eps={eps}")
    y, sp, sc, res, g = _inputs(50, 8, 2048, 400, seed=99, scale=1e-3)
    _check(orc, y, sp, sc, res, g, eps)
    y, sp, sc, res, g = _inputs(50, 8, 2048, 400, seed=98, scale=1e3)
    _check(orc, y, sp, sc, res, g, eps)


def test_fused_norm_no_expert_rows(orc):
    # n_y == 0: every route skipped, x is the residual itself
    note("combine_add_rmsnorm n_y=0")
    y, sp, sc, res, g = _inputs(21, 8, 1024, 0, seed=5)
    _check(orc, y, sp, sc, res, g, 1e-6)


def test_fused_norm_matches_combine(orc):
    # x_out equals mep_combine's output on a zero residual
    torch = require_gpu()
    import combine_balancing_amd as cba
    note("combine_add_rmsnorm vs combine")
    y, sp, sc, res, g = _inputs(64, 8, 7168, 512, seed=8)
    zero = np.zeros_like(res)
    _, xo, _ = cba.combine_add_rmsnorm(dev(y), dev(sp), dev(sc), dev(zero), dev(g))
    ob, _ = cba.combine(dev(y), dev(sp), dev(sc), out_bf16=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(xo), host(ob))


def test_fused_norm_headline_shape(orc):
    # S=4096 K=8 H=7168 on rank 0's planned send map: every token (x_out bit
    # for bit, rstd and y within the bounds above)
    torch = require_gpu()
    note("combine_add_rmsnorm dsv3")
    d = synth.make_plan_inputs("dsv3")
    R, E, S, K = d["R"], d["E"], d["S"], d["K"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    rng = np.random.default_rng(44)
    res = synth.bf16_normal(rng, (S, d["H"]))
    g = synth.bf16_normal(rng, (d["H"],))
    _check(orc, d["y_ret"], p["send_pos"], d["scores"][0], res, g, 1e-6)
    del torch


def test_fused_norm_random_shapes(orc):
    """Twenty seeded shapes (T up to 300, K up to 16, H up to 16384, few or
    no expert rows, pruned routes, residuals over a range of magnitudes,
    three eps values), every token checked."""
    require_gpu()
    shapes = np.random.default_rng(20261208)
    for case in range(20):
        T = int(shapes.integers(1, 301))
        K = int(shapes.integers(1, 17))
        H = 8 * int(shapes.integers(1, 2049))
        n_y = int(shapes.integers(0, 3 * T * K + 1)) if shapes.random() < 0.9 else 0
        eps = float(shapes.choice([0.0, 1e-6, 1e-2]))
        scale = float(2.0 ** shapes.integers(-6, 7))
        prune = float(shapes.choice([0.0, 0.15, 0.6]))
        note(f"combine_add_rmsnorm random case {case}: T={T} K={K} H={H} n_y={n_y} eps={eps}")
        y, sp, sc, res, g = _inputs(T, K, H, n_y, 1000 + case, prune=prune, scale=scale)
        _check(orc, y, sp, sc, res, g, eps)
