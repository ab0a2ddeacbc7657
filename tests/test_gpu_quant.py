"""GPU parity of mep_dispatch_quant (int8 dispatch) against the oracle.

Both sides start from the same byte fill, so whole message buffers are
compared bit for bit: the codes and scales written, and the bytes neither
side writes. The quantization decision (rint of an fp32 quotient) is taken
in fp32 on both sides.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

FILL = 0x5A


def _run(orc, x, sp, K, smooth=None, ex=None, n_rows=None):
    torch = require_gpu()
    import combine_balancing_amd as cba
    T, H = x.shape
    n_rows = T * K if n_rows is None else n_rows
    mb = orc.quant_msg_bytes(H)
    assert cba.quant_msg_bytes(H) == mb
    ref = np.full((n_rows, mb), FILL, np.uint8)
    orc.dispatch_quant(x, sp, K, smooth=smooth, route_expert=ex, n_rows=n_rows, msgs=ref)
    msgs = torch.full((n_rows, mb), FILL, dtype=torch.uint8, device="cuda")
    cba.dispatch_quant(K, dev(x), dev(sp), send_msgs=msgs,
                       smooth=None if smooth is None else dev(smooth),
                       route_expert=None if ex is None else dev(ex))
    torch.cuda.synchronize()
    got = host(msgs)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{len(bad)} bytes differ, first at {bad[:4].tolist()}")
    return got


CASES = [(1, 1, 8), (5, 3, 24), (64, 8, 128), (37, 4, 1032), (19, 6, 5120), (40, 8, 7168),
         (7, 2, 16384), (130, 1, 256), (9, 16, 2048)]


@pytest.mark.parametrize("T,K,H", CASES)
def test_quant_shapes(orc, T, K, H):
    note(f"dispatch_quant T={T} K={K} H={H}")
    rng = np.random.default_rng(T * 7 + K * 131 + H)
    x = synth.bf16_normal(rng, (T, H))
    sp = rng.permutation(T * K).astype(np.int32)
    sp[rng.random(T * K) < 0.1] = -1
    _run(orc, x, sp, K)


@pytest.mark.parametrize("T,K,H", [(33, 4, 512), (21, 8, 7168), (5, 2, 16384)])
def test_quant_smoothing(orc, T, K, H):
    note(f"dispatch_quant smoothing T={T} K={K} H={H}")
    rng = np.random.default_rng(T + K + H)
    E = 6
    x = synth.bf16_normal(rng, (T, H))
    sm = (rng.random((E, H), dtype=np.float32) * 2.0 + 0.1).astype(np.float32)
    ex = rng.integers(0, E, T * K).astype(np.int32)
    ex[::5] = E  # no such expert: skipped on both sides
    sp = rng.permutation(T * K).astype(np.int32)
    _run(orc, x, sp, K, smooth=sm, ex=ex)


def test_quant_rounding_edges(orc):
    # ties to even on the GPU (s = 1 exactly), a zero row, a tiny row
    note("dispatch_quant rounding edges")
    row = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 1.5, -127.0, 0.0], np.float32)
    x = np.zeros((3, 8), np.uint16)
    x[0] = (row.view(np.uint32) >> 16).astype(np.uint16)
    x[2] = (np.full(8, 1e-30, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = _run(orc, x, np.array([0, 1, 2], np.int32), 1)
    assert list(got[0, :8].view(np.int8)) == [127, 2, 4, -2, 0, 2, -127, 0]
    assert np.all(got[1, :8] == 0)


def test_quant_quotient_next_to_half_step(orc):
    # rows whose v / s lands next to 63.5, where the IEEE division (63, then
    # 64 for a quotient that rounds onto the tie) differs from a product
    # with a rounded reciprocal and from an fp64 quotient; the values
    # expected are those of the oracle's pin, from exact rationals
    note("dispatch_quant quotient next to a half step")
    rows = np.array([[1.3671875, 0.68359375] + [0.0] * 6, [1.1875, 0.59375] + [0.0] * 6,
                     [-1.3671875, -0.68359375] + [0.0] * 6], np.float32)
    x = (rows.view(np.uint32) >> 16).astype(np.uint16)
    got = _run(orc, x, np.array([0, 1, 2], np.int32), 1)
    assert list(got[:, 1].view(np.int8)) == [63, 64, -63]


def test_quant_subnormal_rows(orc):
    # bf16 subnormal rows: quantized like any other (s stays a nonzero
    # subnormal), and, smoothed down to a few smallest fp32 subnormals, a
    # scale that rounds to zero giving all-zero codes
    note("dispatch_quant subnormal rows")
    x = np.zeros((3, 16), np.uint16)
    x[0, :4] = [0x0001, 0x8002, 0x0004, 0x007F]
    x[1, :3] = [0x0001, 0x8001, 0x0003]
    x[2, :5] = [0x0080, 0x8100, 0x0001, 0x0040, 0x80FF]  # normals and subnormals mixed
    got = _run(orc, x, np.array([0, 1, 2], np.int32), 1)
    assert list(got[0, :4].view(np.int8)) == [1, -2, 4, 127]
    sm = np.ones((2, 16), np.float32)
    sm[1] = 2.0 ** -12
    ex = np.array([0, 1, 0], np.int32)
    got = _run(orc, x, np.array([0, 1, 2], np.int32), 1, smooth=sm, ex=ex)
    assert np.all(got[1, :16] == 0)


def test_quant_headline_shape_and_grouping(orc):
    # S=4096 K=8 H=7168 on rank 0's planned send map: every message byte;
    # then the receive grouping of message rows (a byte copy) vs the oracle's
    torch = require_gpu()
    import combine_balancing_amd as cba
    note("dispatch_quant dsv3")
    d = synth.make_plan_inputs("dsv3", stand_ins=False)
    R, E, S, K, H, C = d["R"], d["E"], d["S"], d["K"], d["H"], d["C"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    msgs = _run(orc, d["x"], p["send_pos"], K)
    note("group int8 messages dsv3")
    raw = msgs.view(np.uint16)  # rows of msg_bytes / 2 units
    _, grouped = cba.dispatch(K, recv_raw=dev(raw), recv_pos=dev(p["recv_pos"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(grouped), orc.group(raw, p["recv_pos"]))


def test_quant_empty():
    torch = require_gpu()
    import combine_balancing_amd as cba
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    sp = torch.zeros(0, dtype=torch.int32, device="cuda")
    m = cba.dispatch_quant(4, x, sp)
    torch.cuda.synchronize()
    assert m.shape[0] == 0


@pytest.mark.parametrize("n,H,n_msgs", [(1, 8, 1), (37, 136, 40), (300, 2048, 320), (64, 7168, 64)])
def test_group_quant_shapes(orc, n, H, n_msgs):
    torch = require_gpu()
    import combine_balancing_amd as cba
    note(f"group_quant n={n} H={H}")
    rng = np.random.default_rng(n + H)
    x = synth.bf16_normal(rng, (n_msgs, H))
    msgs = orc.dispatch_quant(x, np.arange(n_msgs, dtype=np.int32), 1)
    rp = rng.integers(0, n_msgs, n).astype(np.int32)
    rp[::9] = -1  # leaves the row untouched
    xq = torch.full((n, H), 7, dtype=torch.int8, device="cuda")
    sc = torch.full((n,), 3.0, dtype=torch.float32, device="cuda")
    cba.group_quant(dev(msgs), dev(rp), H, x_q=xq, scales=sc)
    torch.cuda.synchronize()
    rxq = np.full((n, H), 7, np.uint8)
    rsc = np.full(n, 3.0, np.float32)
    gx, gs = orc.group_quant(msgs, rp, H)
    ok = rp >= 0
    rxq[ok], rsc[ok] = gx[ok], gs[ok]
    assert np.array_equal(host(xq).view(np.uint8), rxq)
    assert np.array_equal(host(sc), rsc)


def test_int8_path_headline(orc):
    # dsv3 rank 0: quantized pack -> (alltoallv stand-in: rank 0's own
    # messages as the arrival buffer) -> receive-side split, vs the oracle
    torch = require_gpu()
    import combine_balancing_amd as cba
    note("int8 path dsv3")
    d = synth.make_plan_inputs("dsv3", stand_ins=False)
    R, E, S, K, H = d["R"], d["E"], d["S"], d["K"], d["H"]
    p = orc.plan(d["topk_ids"], R, E, S, K, m=0)
    sp, rp = dev(p["send_pos"]), dev(p["recv_pos"])
    msgs = cba.dispatch_quant(K, dev(d["x"]), sp)
    xq, sc = cba.group_quant(msgs, rp, H)
    torch.cuda.synchronize()
    ref_m = orc.dispatch_quant(d["x"], p["send_pos"], K)
    gx, gs = orc.group_quant(ref_m, p["recv_pos"], H)
    assert np.array_equal(host(xq).view(np.uint8), gx)
    assert np.array_equal(host(sc), gs)


def test_quant_random_shapes(orc):
    """Twenty-four seeded shapes (T up to 300, K up to 16, H up to 16384,
    rows scaled over a wide range of magnitudes), half of them smoothed with
    some routes naming no expert; then the receive split of the messages."""
    torch = require_gpu()
    import combine_balancing_amd as cba
    shapes = np.random.default_rng(20261207)
    for case in range(24):
        T = int(shapes.integers(1, 301))
        K = int(shapes.integers(1, 17))
        H = 8 * int(shapes.integers(1, 2049))
        smooth = bool(shapes.random() < 0.5)
        rng = np.random.default_rng(case)
        x = synth.bf16_normal(rng, (T, H))
        mag = np.float32(2.0) ** rng.integers(-20, 21, T).astype(np.float32)
        xf = (x.astype(np.uint32) << 16).view(np.float32)
        x = synth.bf16_from_f32_trunc(xf * mag[:, None])
        sp = rng.permutation(T * K).astype(np.int32)
        sp[rng.random(T * K) < 0.1] = -1
        sm = ex = None
        if smooth:
            E = int(rng.integers(1, 13))
            sm = (rng.random((E, H), dtype=np.float32) * 2.0 + 0.05).astype(np.float32)
            ex = rng.integers(0, E + 1, T * K).astype(np.int32)  # E: no such expert
        note(f"dispatch_quant random case {case}: T={T} K={K} H={H} smooth={smooth}")
        msgs = _run(orc, x, sp, K, smooth=sm, ex=ex)
        n = int(rng.integers(1, min(2 * T * K, 2000) + 1))
        rp = rng.integers(-1, T * K, n).astype(np.int32)
        xq = torch.full((n, H), 7, dtype=torch.int8, device="cuda")
        sc = torch.full((n,), 3.0, dtype=torch.float32, device="cuda")
        cba.group_quant(dev(msgs), dev(rp), H, x_q=xq, scales=sc)
        torch.cuda.synchronize()
        rxq = np.full((n, H), 7, np.uint8)
        rsc = np.full(n, 3.0, np.float32)
        gx, gs = orc.group_quant(msgs, rp, H)
        ok = rp >= 0
        rxq[ok], rsc[ok] = gx[ok], gs[ok]
        assert np.array_equal(host(xq).view(np.uint8), rxq), f"case {case}"
        assert np.array_equal(host(sc), rsc), f"case {case}"
