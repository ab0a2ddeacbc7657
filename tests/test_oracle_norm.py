"""Pins of the oracle's combine + residual add + RMSNorm.

The pages ("aclnnMoeUpdateExpert" op doc, call example) name the fused
combine variant's extra tensors (residual x, gamma; outputs y, rstd and the
summed x) without a formula; the oracle takes the usual add + RMSNorm of the
unrounded fp32 sum. These pins fix that reading by a hand example, exact
special cases and invariants, and tie the combine part to the pinned
oracle_combine.
"""
import numpy as np
import pytest

import synth


def _bf16(v):
    a = np.asarray(v, np.float32)
    assert np.all((a.view(np.uint32) & 0xFFFF) == 0), "value must be exact in bf16"
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _pruned(T, K):
    return np.full(T * K, -1, np.int32)


def test_hand_example(orc):
    # x = [1, 2, 2, 4]: sum of squares 25, mean 6.25, rstd = 1/2.5 = 0.4;
    # y = x * 0.4 * gamma with gamma = [1, 0.5, 2, 1] -> [0.4, 0.4, 1.6, 1.6]
    y_ret = np.zeros((1, 4), np.uint16)
    res = _bf16([[1.0, 2.0, 2.0, 4.0]])
    g = _bf16([1.0, 0.5, 2.0, 1.0])
    o = orc.combine_add_rmsnorm(y_ret, _pruned(1, 2), np.ones((1, 2), np.float32), res, g, 0.0)
    assert np.array_equal(o["x_out"], res)
    assert abs(o["rstd"][0] - 0.4) < 1e-15
    assert np.allclose(o["y"][0], [0.4, 0.4, 1.6, 1.6], rtol=1e-15, atol=0)


def test_zero_row_gives_rsqrt_eps(orc):
    # all-zero sum: rstd = 1/sqrt(eps) (eps inside the root), y = 0
    T, H = 3, 16
    o = orc.combine_add_rmsnorm(np.zeros((1, H), np.uint16), _pruned(T, 1),
                                np.ones((T, 1), np.float32), np.zeros((T, H), np.uint16),
                                _bf16(np.ones(H)), 1e-6)
    assert np.allclose(o["rstd"], 1e3, rtol=1e-14)
    assert np.all(o["y"] == 0.0)


def test_residual_only_is_exact_copy(orc):
    rng = np.random.default_rng(3)
    T, K, H = 9, 4, 40
    res = synth.bf16_normal(rng, (T, H))
    o = orc.combine_add_rmsnorm(synth.bf16_normal(rng, (5, H)), _pruned(T, K),
                                np.ones((T, K), np.float32), res, _bf16(np.ones(H)), 1e-6)
    assert np.array_equal(o["x_out"], res)
    assert np.array_equal(o["x_f32"], _f32(res))


def test_zero_residual_equals_combine(orc):
    # with a zero residual the summed x is the combine's output bit for bit
    rng = np.random.default_rng(4)
    T, K, H = 32, 8, 64
    y = synth.bf16_normal(rng, (T * K + 3, H))
    sp = rng.permutation(T * K + 3)[: T * K].astype(np.int32)
    sp[rng.random(T * K) < 0.2] = -1
    sc = synth.make_scores(rng, T, K)
    ob, of = orc.combine(y, sp, sc)
    o = orc.combine_add_rmsnorm(y, sp, sc, np.zeros((T, H), np.uint16), _bf16(np.ones(H)), 1e-6)
    assert np.array_equal(o["x_f32"], of)
    assert np.array_equal(o["x_out"], ob)


def test_rows_past_n_y_are_skipped(orc):
    # a route whose row lies at or past the n_y returned rows adds nothing,
    # as a route with position -1 does
    rng = np.random.default_rng(6)
    T, K, H, n_y = 9, 4, 32, 20
    y = synth.bf16_normal(rng, (n_y, H))
    sp = rng.integers(0, n_y, T * K).astype(np.int32)
    sc = synth.make_scores(rng, T, K)
    res = synth.bf16_normal(rng, (T, H))
    g = _bf16(np.ones(H))
    far = sp.copy()
    far[::3] = n_y + np.arange(far[::3].size)
    drop = sp.copy()
    drop[::3] = -1
    a = orc.combine_add_rmsnorm(y, far, sc, res, g, 1e-6, n_y=n_y)
    b = orc.combine_add_rmsnorm(y, drop, sc, res, g, 1e-6, n_y=n_y)
    for key in ("x_out", "x_f32", "rstd", "y"):
        assert np.array_equal(a[key], b[key]), key


def test_unit_rms_when_eps_zero(orc):
    # eps = 0: sum_h (y/gamma)^2 / H = 1 for every row
    rng = np.random.default_rng(5)
    T, K, H = 16, 2, 96
    y = synth.bf16_normal(rng, (T * K, H))
    sp = rng.permutation(T * K).astype(np.int32)
    g = synth.bf16_normal(rng, (H,))
    g[g == 0] = _bf16([1.0])[0]
    o = orc.combine_add_rmsnorm(y, sp, synth.make_scores(rng, T, K),
                                synth.bf16_normal(rng, (T, H)), g, 0.0)
    q = (o["y"] / _f32(g).astype(np.float64)[None, :]) ** 2
    assert np.allclose(q.mean(axis=1), 1.0, rtol=0, atol=1e-12)


def test_scale_invariance_is_exact(orc):
    # doubling every expert row and the residual doubles x exactly (powers of
    # two scale fp32 products and sums exactly), so with eps = 0 rstd halves
    # exactly and y is unchanged bit for bit
    rng = np.random.default_rng(6)
    T, K, H = 12, 4, 48
    y = synth.bf16_normal(rng, (T * K, H))
    res = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    sc = synth.make_scores(rng, T, K)
    g = synth.bf16_normal(rng, (H,))

    def twice(b):
        return _bf16(_f32(b) * np.float32(2.0))

    a = orc.combine_add_rmsnorm(y, sp, sc, res, g, 0.0)
    b = orc.combine_add_rmsnorm(twice(y), sp, sc, twice(res), g, 0.0)
    assert np.array_equal(b["x_f32"], a["x_f32"] * np.float32(2.0))
    assert np.array_equal(b["rstd"], a["rstd"] / 2.0)
    assert np.array_equal(b["y"], a["y"])


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_eps_enters_under_the_root(orc, eps):
    # constant row c: rstd = 1/sqrt(c^2 + eps) (closed form)
    H = 8
    for c in (0.5, 3.0, -2.0):
        o = orc.combine_add_rmsnorm(np.zeros((1, H), np.uint16), _pruned(1, 1),
                                    np.ones((1, 1), np.float32), _bf16(np.full((1, H), c)),
                                    _bf16(np.ones(H)), eps)
        assert abs(o["rstd"][0] - 1.0 / np.sqrt(c * c + eps)) <= 1e-15 * o["rstd"][0]
        assert np.allclose(o["y"], c / np.sqrt(c * c + eps), rtol=1e-15, atol=0)
