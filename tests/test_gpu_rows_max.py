"""Pack, combine and receive grouping at the largest flat size the library
accepts: T * H/8 = 2^31 - H/8 vectors (H = 8192, T = 2^21 - 1, K = 1), so the
flat kernels' 32-bit thread index runs up to just below 2^31.

Every output row is checked, on the device with torch's own gather and
compare, a 2 GiB block at a time (each buffer is 32 GiB). With K = 1 and
unit scores, combine returns each token's row exactly: its values are normal
bf16 numbers, so 0 + 1.0 * y is y in fp32 and rounds back to the same bf16.
"""
import pytest

from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

H = 8192
NVEC = H // 8
T = (1 << 31) // NVEC - 1  # T * NVEC = 2^31 - NVEC, the largest below 2^31
BLOCK = 1 << 17             # rows per checking block (2 GiB)


def _rows_equal(torch, a, b, ctx):
    for r0 in range(0, T, BLOCK):
        r1 = min(T, r0 + BLOCK)
        if not torch.equal(a(r0, r1), b(r0, r1)):
            raise AssertionError(f"{ctx}: rows {r0}..{r1 - 1} differ")


def test_row_movers_at_largest_flat_size():
    torch = require_gpu()
    import combine_balancing_amd as cba
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 110 * (1 << 30):
        pytest.skip("needs about 100 GiB of free device memory")
    note(f"row movers at the flat limit: T={T} H={H} K=1")
    g = torch.Generator(device="cuda")
    g.manual_seed(20261203)
    # bf16 patterns: random sign and 8 low bits, exponent 126 or 127, so
    # every value is a normal number in [0.5, 2)
    x = torch.randint(-32768, 32767, (T, H), dtype=torch.int16, device="cuda", generator=g)
    x.bitwise_and_(-32513)  # 0x80FF
    x.bitwise_or_(0x3F00)
    send_pos = torch.randperm(T, device="cuda", generator=g).to(torch.int32)
    sp = send_pos.long()

    send_buf = torch.empty(T, H, dtype=torch.int16, device="cuda")
    cba.dispatch(1, x=x, send_pos=send_pos, send_buf=send_buf)
    torch.cuda.synchronize()
    _rows_equal(torch, lambda a, b: send_buf[sp[a:b]], lambda a, b: x[a:b], "pack")

    out = torch.empty(T, H, dtype=torch.int16, device="cuda")
    scores = torch.ones(T, 1, dtype=torch.float32, device="cuda")
    cba.combine(send_buf, send_pos, scores, out_bf16=out)
    torch.cuda.synchronize()
    _rows_equal(torch, lambda a, b: out[a:b], lambda a, b: x[a:b], "combine")
    del out

    grouped = torch.empty(T, H, dtype=torch.int16, device="cuda")
    cba.dispatch(1, recv_raw=send_buf, recv_pos=send_pos, recv_grouped=grouped)
    torch.cuda.synchronize()
    _rows_equal(torch, lambda a, b: grouped[a:b], lambda a, b: x[a:b], "group")
    del x, send_buf, grouped, sp, send_pos
    torch.cuda.empty_cache()  # hand the ~96 GiB back before the next test
