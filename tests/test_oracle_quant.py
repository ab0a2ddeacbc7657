"""Pins of the oracle's int8 dispatch (dynamic quantization of routed rows).

The pages ("aclnnMoeDistributeDispatchSetup" op doc) fix the message size,
Align512(Align32(H) + 4) bytes, and say token data may be quantized
dynamically, optionally with per-expert smoothing scales; they give no
formula. The oracle reads it as symmetric per-route int8 quantization in
fp32: s = amax / 127, q = rint(v / s). These pins fix that reading by its
defining properties (the largest magnitude maps to +-127, every value is
within half a step, ties go to even, exact behaviour under power-of-two
scaling) and the message layout.
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


def _q(msgs, H):
    return msgs[:, :H].view(np.int8).astype(np.int32)


def _s(msgs, H):
    hq = (H + 31) // 32 * 32
    return np.ascontiguousarray(msgs[:, hq:hq + 4]).view(np.float32).reshape(-1)


@pytest.mark.parametrize("H,size", [(7168, 7680), (100, 512), (2048, 2560), (508, 1024), (480, 512), (512, 1024)])
def test_message_size(orc, H, size):
    assert orc.quant_msg_bytes(H) == size


def test_layout_and_untouched_bytes(orc):
    # H = 100: values in bytes [0,100), scale at [128,132); the rest untouched
    rng = np.random.default_rng(1)
    x = synth.bf16_normal(rng, (3, 100))
    msgs = np.full((6, 512), 0xAB, np.uint8)
    sp = np.array([0, 2, 4, 5, 1, 3], np.int32)
    orc.dispatch_quant(x, sp, 2, msgs=msgs)
    assert np.all(msgs[:, 100:128] == 0xAB)
    assert np.all(msgs[:, 132:] == 0xAB)
    assert np.all(_s(msgs, 100) > 0)


def test_ties_to_even_and_extremes(orc):
    # amax = 127 gives s = 1 exactly; 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, -0.5 -> 0
    x = _bf16([[127.0, 2.5, 3.5, -2.5, -0.5, 1.5, -127.0, 0.0]])
    m = orc.dispatch_quant(x, np.array([0], np.int32), 1)
    assert _s(m, 8)[0] == 1.0
    assert list(_q(m, 8)[0]) == [127, 2, 4, -2, 0, 2, -127, 0]


def test_max_maps_to_127_and_half_step_bound(orc):
    rng = np.random.default_rng(2)
    T, K, H = 40, 3, 256
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    m = orc.dispatch_quant(x, sp, K)
    q, s = _q(m, H), _s(m, H)
    for t in range(T):
        v = _f32(x[t]).astype(np.float64)
        for k in range(K):
            r = sp[t * K + k]
            j = np.argmax(np.abs(v))
            assert abs(q[r, j]) == 127 and np.sign(q[r, j]) == np.sign(v[j])
            assert s[r] == np.float32(np.float32(np.abs(v).max()) / np.float32(127.0))
            # half a step, plus the fp32 rounding of v / s (|v / s| <= 127,
            # so at most 127 * 2^-24 steps)
            err = np.abs(q[r] * np.float64(s[r]) - v)
            assert np.all(err <= (0.5 + 127 * 2.0 ** -24) * s[r] + 1e-30)


def test_zero_row(orc):
    x = np.zeros((2, 64), np.uint16)
    m = orc.dispatch_quant(x, np.array([1, 0], np.int32), 1)
    assert np.all(m[:, :64] == 0) and np.all(_s(m, 64) == 0.0)


def test_power_of_two_scaling_is_exact(orc):
    rng = np.random.default_rng(3)
    x = synth.bf16_normal(rng, (16, 96))
    x2 = _bf16(_f32(x) * np.float32(4.0))
    sp = np.arange(16, dtype=np.int32)
    a = orc.dispatch_quant(x, sp, 1)
    b = orc.dispatch_quant(x2, sp, 1)
    assert np.array_equal(_q(a, 96), _q(b, 96))
    assert np.array_equal(_s(b, 96), _s(a, 96) * np.float32(4.0))


def test_smoothing(orc):
    # all-ones smoothing equals none; a power-of-two smoothing row of one
    # expert equals scaling that route's row
    rng = np.random.default_rng(4)
    T, K, H, E = 12, 2, 64, 5
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    ex = rng.integers(0, E, T * K).astype(np.int32)
    plain = orc.dispatch_quant(x, sp, K)
    ones = orc.dispatch_quant(x, sp, K, smooth=np.ones((E, H), np.float32), route_expert=ex)
    assert np.array_equal(plain, ones)
    sm = np.ones((E, H), np.float32)
    sm[2] = 2.0
    got = orc.dispatch_quant(x, sp, K, smooth=sm, route_expert=ex)
    q, s, qp, spl = _q(got, H), _s(got, H), _q(plain, H), _s(plain, H)
    for f in range(T * K):
        r = sp[f]
        assert np.array_equal(q[r], qp[r])
        assert s[r] == (spl[r] * np.float32(2.0) if ex[f] == 2 else spl[r])


def test_smoothing_per_column_and_expert(orc):
    # each route reads its own expert's smoothing row, column by column: with
    # power-of-two factors the product is exact, so a smoothed route's
    # message equals the unsmoothed message of its row pre-multiplied
    rng = np.random.default_rng(5)
    T, K, H, E = 10, 3, 48, 4
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    ex = rng.integers(0, E, T * K).astype(np.int32)
    h, e = np.meshgrid(np.arange(H), np.arange(E))
    sm = np.exp2(((h * 3 + e * 2) % 7 - 3).astype(np.float32)).astype(np.float32)
    got = orc.dispatch_quant(x, sp, K, smooth=sm, route_expert=ex)
    for f in range(T * K):
        t, r = f // K, sp[f]
        row = _bf16(_f32(x[t]) * sm[ex[f]])
        ref = orc.dispatch_quant(row[None, :], np.array([0], np.int32), 1)
        assert np.array_equal(got[r], ref[0]), f


def test_smoothing_skips_routes_without_an_expert(orc):
    # with smoothing, a route whose expert id is outside [0, E) has no
    # smoothing row: it is skipped and its message row left untouched
    rng = np.random.default_rng(7)
    T, K, H, E = 5, 2, 32, 3
    x = synth.bf16_normal(rng, (T, H))
    sp = np.arange(T * K, dtype=np.int32)
    ex = rng.integers(0, E, T * K).astype(np.int32)
    ex[[1, 6]] = [E, -1]
    sm = np.full((E, H), 2.0, np.float32)
    msgs = np.full((T * K, orc.quant_msg_bytes(H)), 0x5A, np.uint8)
    got = orc.dispatch_quant(x, sp, K, smooth=sm, route_expert=ex, msgs=msgs)
    assert np.all(got[[1, 6]] == 0x5A)
    ok = np.setdiff1d(np.arange(T * K), [1, 6])
    assert not np.any(np.all(got[ok] == 0x5A, axis=1))


def test_scale_that_underflows_gives_zero_codes(orc):
    # s = fl(amax / 127) is zero for a nonzero row when amax is a few
    # smallest subnormals (here bf16 2^-133 smoothed by 2^-12: v = 2^-145,
    # and 2^-145 / 127 rounds to +0); with s = 0 every code is 0, as for a
    # zero row, and the scale written is +0
    x = np.zeros((1, 8), np.uint16)
    x[0, :3] = [0x0001, 0x8001, 0x0003]  # 2^-133, -2^-133, 3 * 2^-133
    sm = np.full((1, 8), 2.0 ** -12, np.float32)
    m = orc.dispatch_quant(x, np.array([0], np.int32), 1, smooth=sm,
                           route_expert=np.zeros(1, np.int32))
    assert np.all(_q(m, 8) == 0)
    assert _s(m, 8)[0] == 0.0 and not np.signbit(_s(m, 8)[0])


def test_subnormal_rows(orc):
    # a row of bf16 subnormals quantizes like any other: its largest
    # magnitude maps to +-127 (s = fl(amax / 127) stays a nonzero subnormal)
    x = np.zeros((1, 8), np.uint16)
    x[0, :4] = [0x0001, 0x8002, 0x0004, 0x007F]  # k * 2^-133
    m = orc.dispatch_quant(x, np.array([0], np.int32), 1)
    s = _s(m, 8)[0]
    assert s > 0.0 and s < np.finfo(np.float32).tiny
    q = _q(m, 8)[0]
    assert q[3] == 127
    assert s == np.float32(2.0 ** -133)  # 127 * 2^-133 / 127, exact
    assert list(q[:3]) == [1, -2, 4]


def _rn32(q):
    """IEEE round-to-nearest-even of a positive rational to fp32 (normal
    range), from the definition: scale into [2^23, 2^24), round the
    integer part half to even."""
    from fractions import Fraction
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return Fraction(round(q / Fraction(2) ** (e - 23))) * Fraction(2) ** (e - 23)


def test_quotient_is_the_correctly_rounded_division(orc):
    # q = rint(fl(v / s)) with fl the IEEE division. The rows below put v / s
    # next to 63.5, where the reading's division and two plausible
    # alternatives disagree. Expected values come from exact rationals.
    from fractions import Fraction
    rows = [[1.3671875, 0.68359375], [1.1875, 0.59375]]
    x = _bf16(np.array([r + [0.0] * 6 for r in rows], np.float32))
    m = orc.dispatch_quant(x, np.array([0, 1], np.int32), 1)
    q, s = _q(m, 8), _s(m, 8)
    for i, (amax, v) in enumerate(rows):
        S = _rn32(Fraction(amax) / 127)
        Q = _rn32(Fraction(v) / S)
        assert s[i] == float(S)
        assert list(q[i][:2]) == [127, round(Q)]
        # the case tells the division apart from a product with a rounded
        # reciprocal and from an unrounded (fp64) quotient
        recip = round(_rn32(Fraction(v) * _rn32(1 / S)))
        exact = round(Fraction(v) / S)
        assert round(Q) != recip
        assert i == 0 or round(Q) != exact
    assert list(q[:, 1]) == [63, 64]


def test_token_copies_identical_and_skips(orc):
    rng = np.random.default_rng(5)
    T, K, H = 10, 4, 48
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    sp[::7] = -1
    msgs = np.full((T * K, orc.quant_msg_bytes(H)), 0x5A, np.uint8)
    orc.dispatch_quant(x, sp, K, msgs=msgs)
    written = set(sp[sp >= 0].tolist())
    for r in range(T * K):
        if r not in written:
            assert np.all(msgs[r] == 0x5A)
    for t in range(T):
        rows = [sp[t * K + k] for k in range(K) if sp[t * K + k] >= 0]
        for r in rows[1:]:
            assert np.array_equal(msgs[r, :H], msgs[rows[0], :H])


def test_group_quant_is_grouping_then_split(orc):
    # the receive-side split equals the (pinned) row grouping of whole
    # messages followed by reading the code bytes and the scale field
    rng = np.random.default_rng(6)
    T, K, H = 30, 4, 200
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    msgs = orc.dispatch_quant(x, sp, K)
    rp = rng.permutation(T * K).astype(np.int32)
    xq, sc = orc.group_quant(msgs, rp, H)
    g = orc.group(msgs.view(np.uint16), rp).view(np.uint8)
    assert np.array_equal(xq, g[:, :H])
    assert np.array_equal(sc, _s(g, H))
    # dequantized rows stay within half a step of the token rows they came from
    tok = np.empty(T * K, np.int64)
    tok[sp] = np.arange(T * K) // K
    for t in range(T * K):
        v = _f32(x[tok[rp[t]]]).astype(np.float64)
        err = np.abs(xq[t].view(np.int8) * np.float64(sc[t]) - v)
        assert np.all(err <= (0.5 + 127 * 2.0 ** -24) * sc[t] + 1e-30)
