"""The C-ABI library: it loads, exports every function include/mep.h
declares, and rejects bad arguments on the host before touching the GPU.

No compute call is made here (no GPU is needed).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mep.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mep_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def B():
    from combine_balancing_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from combine_balancing_amd import build
        build.build()
    _binding.lib()
    return _binding


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("mep_plan", "mep_remap_prune", "mep_dispatch", "mep_combine",
              "mep_plan_workspace_size", "mep_status_str", "mep_version",
              "mep_dispatch_to_peers", "mep_combine_from_peers", "mep_ungroup",
              "mep_combine_add_rmsnorm", "mep_quant_msg_bytes", "mep_dispatch_quant",
              "mep_group_quant", "mep_plan_weight_rows", "mep_plan_dedup_workspace_size",
              "mep_plan_dedup", "mep_plan_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mep_[a-z_]+)\b", out))
    assert set(_declared()) <= exported


def test_library_has_gfx950_code(B):
    # the offload bundle embedded in the library names its one target
    data = open(B.LIB_PATH, "rb").read()
    assert b"__CLANG_OFFLOAD_BUNDLE__" in data
    assert b"amdgcn-amd-amdhsa--gfx950" in data
    assert b"gfx942" not in data and b"sm_" + b"90" not in data


def test_status_strings(B):
    assert B.status_str(0) == "MEP_OK"
    for c in range(1, 5):
        assert B.status_str(c).startswith("MEP_ERR")
    assert B.lib().mep_version() >= 100


def test_workspace_size(B):
    assert B.mep_plan_workspace_size(8, 256, 4096, 8) > 8 * 256 * 4
    assert B.mep_plan_workspace_size(0, 256, 4096, 8) == 0
    assert B.mep_plan_workspace_size(8, 2000, 4096, 8) == 0   # E > 1024
    assert B.mep_plan_workspace_size(8, 4, 16, 8) == 0       # K > E
    assert B.mep_plan_workspace_size(2048, 256, 16, 8) == 0  # R > 1024
    # every rank count up to the limit has a chunking (one chunk per source
    # at least), from tiny to large route counts
    for R in (1, 511, 512, 513, 1024):
        for S, K in ((1, 1), (3, 2), (8192, 8)):
            assert B.mep_plan_workspace_size(R, 256, S, K) > 0 or R * S * K > (1 << 30)
    assert B.mep_plan_workspace_size(1024, 1024, 1 << 17, 16) == 0  # N > 2^30


def _plan(B, R=8, E=256, S=16, K=8, m=0, ids=1, ws=256, wsb=1 << 30, outs=1, rd=1, rs=1):
    o = [outs] * 12
    o[2], o[3] = rd, rs
    return B.mep_plan(R, E, S, K, m, ids, ws, wsb, *o, None)


def test_plan_validation(B):
    assert _plan(B, ids=None) == B.MEP_ERR_NULLPTR
    assert _plan(B, outs=None, rd=1, rs=1) == B.MEP_ERR_NULLPTR
    assert _plan(B, R=0) == B.MEP_ERR_SHAPE
    assert _plan(B, E=1025) == B.MEP_ERR_SHAPE
    assert _plan(B, K=300) == B.MEP_ERR_PARAM
    assert _plan(B, m=8) == B.MEP_ERR_PARAM
    assert _plan(B, m=-1) == B.MEP_ERR_PARAM
    assert _plan(B, wsb=16) == B.MEP_ERR_PARAM
    assert _plan(B, ws=258) == B.MEP_ERR_PARAM      # misaligned workspace
    assert _plan(B, rd=None) == B.MEP_ERR_PARAM     # route maps come in pairs


def _remap(B, BS=4, K=2, E=8, F=3, ws=4, ppr=2, rank=0, mode=0, ids=1, table=1, sc=None,
           sdt=1, thr=None, act=None, bal=1, mask=1, sp=None, scnt=None):
    return B.mep_remap_prune(BS, K, E, F, ws, ppr, rank, mode, ids, table, sc, sdt, thr, act,
                             bal, mask, sp, scnt, None)


def test_remap_validation(B):
    assert _remap(B, ids=None) == B.MEP_ERR_NULLPTR
    assert _remap(B, mask=None) == B.MEP_ERR_NULLPTR
    assert _remap(B, mode=2) == B.MEP_ERR_PARAM
    assert _remap(B, sc=16) == B.MEP_ERR_PARAM              # scales without threshold
    assert _remap(B, thr=16) == B.MEP_ERR_PARAM             # threshold without scales
    assert _remap(B, act=16) == B.MEP_ERR_PARAM             # mask without scales
    assert _remap(B, sp=16) == B.MEP_ERR_PARAM              # send map needs both
    assert _remap(B, sc=16, thr=16, sdt=7) == B.MEP_ERR_PARAM
    assert _remap(B, rank=4) == B.MEP_ERR_PARAM             # mode 0 rank out of range
    assert _remap(B, K=17) == B.MEP_ERR_SHAPE
    assert _remap(B, K=9, E=8) == B.MEP_ERR_PARAM
    assert _remap(B, F=6, ws=4) == B.MEP_ERR_SHAPE          # F > world_size + 1
    assert _remap(B, F=1) == B.MEP_ERR_SHAPE
    assert _remap(B, ws=600, ppr=2) == B.MEP_ERR_SHAPE      # > 1024 instances
    assert _remap(B, BS=0) == B.MEP_ERR_SHAPE
    assert _remap(B, BS=513) == B.MEP_ERR_SHAPE             # op doc limit BS <= 512
    assert _remap(B, E=1025) == B.MEP_ERR_SHAPE


def test_dispatch_combine_validation(B):
    D = B.mep_dispatch
    assert D(4, 2, 64, None, None, None, 8, 0, None, None, 8, None, None) == B.MEP_ERR_PARAM
    assert D(0, 2, 64, None, None, None, 8, 0, None, None, 8, None, None) == B.MEP_OK
    assert D(4, 2, 64, 16, None, 16, 8, 0, None, None, 8, None, None) == B.MEP_ERR_NULLPTR
    assert D(4, 2, 60, 16, 16, 16, 8, 0, None, None, 8, None, None) == B.MEP_ERR_SHAPE   # H % 8
    assert D(4, 2, 64, 8, 16, 16, 8, 0, None, None, 8, None, None) == B.MEP_ERR_SHAPE    # unaligned
    assert D(4, 65, 64, 16, 16, 16, 8, 0, None, None, 8, None, None) == B.MEP_ERR_SHAPE  # K > 64
    assert D(0, 2, 64, None, None, None, 8, 4, 16, 16, 8, None, None) == B.MEP_ERR_NULLPTR
    assert D(0, 2, 64, None, None, None, 8, -1, 16, 16, 8, 16, None) == B.MEP_ERR_SHAPE
    # buffer row counts: negative sizes are rejected before any launch
    assert D(4, 2, 64, 16, 16, 16, -1, 0, None, None, 0, None, None) == B.MEP_ERR_SHAPE
    assert D(0, 2, 64, None, None, None, 0, 4, 16, 16, -1, 16, None) == B.MEP_ERR_SHAPE
    Cb = B.mep_combine
    assert Cb(0, 2, 64, None, 0, None, None, None, None, None) == B.MEP_OK
    assert Cb(4, 2, 64, None, 8, 16, 16, 16, None, None) == B.MEP_ERR_NULLPTR
    assert Cb(4, 2, 64, 16, 8, 16, 16, None, None, None) == B.MEP_ERR_NULLPTR
    assert Cb(4, 2, 64, 24, 8, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE          # unaligned
    assert Cb(4, 0, 64, 16, 8, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE
    assert Cb(4, 2, 12, 16, 8, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE


def test_package_has_no_fallback(monkeypatch, tmp_path):
    from combine_balancing_amd import _binding
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _binding.lib()


def test_zero_copy_and_ungroup_validation(B):
    P = B.mep_dispatch_to_peers
    assert P(0, 2, 64, 4, 8, None, None, None, None, None) == B.MEP_OK
    assert P(4, 2, 64, 4, 8, None, 16, 16, 16, None) == B.MEP_ERR_NULLPTR
    assert P(4, 2, 60, 4, 8, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert P(4, 2, 64, 0, 8, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert P(4, 2, 64, 1025, 8, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE   # R > 1024
    assert P(4, 2, 64, 4, 8, 8, 16, 16, 16, None) == B.MEP_ERR_SHAPE      # unaligned x
    Q = B.mep_combine_from_peers
    assert Q(0, 2, 64, 4, 8, None, None, None, None, None, None, None) == B.MEP_OK
    assert Q(4, 2, 64, 4, 8, 16, 16, 16, 16, None, None, None) == B.MEP_ERR_NULLPTR
    assert Q(4, 0, 64, 4, 8, 16, 16, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE
    assert Q(4, 2, 64, 1025, 8, 16, 16, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE  # R > 1024
    U = B.mep_ungroup
    assert U(0, 64, None, None, None, None) == B.MEP_OK
    assert U(4, 64, None, 16, 16, None) == B.MEP_ERR_NULLPTR
    assert U(4, 12, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert U(-1, 64, 16, 16, 16, None) == B.MEP_ERR_SHAPE


def test_combine_add_rmsnorm_validation(B):
    f = B.mep_combine_add_rmsnorm
    assert f(0, 2, 64, None, 0, None, None, None, None, 1e-6, None, None, None, None) == B.MEP_OK
    assert f(4, 2, 64, 16, 4, 16, 16, 16, 16, -1.0, None, 16, None, None) == B.MEP_ERR_PARAM
    assert f(4, 2, 64, 16, 4, 16, 16, 16, 16, float("nan"), None, 16, None, None) == B.MEP_ERR_PARAM
    assert f(4, 2, 16392, 16, 4, 16, 16, 16, 16, 1e-6, None, 16, None, None) == B.MEP_ERR_SHAPE
    assert f(4, 2, 60, 16, 4, 16, 16, 16, 16, 1e-6, None, 16, None, None) == B.MEP_ERR_SHAPE
    assert f(4, 2, 64, 16, 4, 16, 16, 16, 16, 1e-6, None, None, None, None) == B.MEP_ERR_NULLPTR
    assert f(4, 2, 64, None, 4, 16, 16, 16, 16, 1e-6, None, 16, None, None) == B.MEP_ERR_NULLPTR
    assert f(4, 2, 64, 16, 4, 16, 16, 8, 16, 1e-6, None, 16, None, None) == B.MEP_ERR_SHAPE


def test_flat_index_limit(B):
    # the flat row kernels index T*(H/8) vectors with 31 bits
    T, H = 1 << 20, 65536
    assert B.mep_dispatch(T, 2, H, 16, 16, 16, 8, 0, None, None, 8, None, None) == B.MEP_ERR_SHAPE
    assert B.mep_combine(T, 2, H, 16, 4, 16, 16, 16, None, None) == B.MEP_ERR_SHAPE
    assert B.mep_dispatch_to_peers(T, 2, H, 2, 8, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE


def test_row_division_by_multiply_is_exact():
    # The row kernels find row = n // d as (n * m) >> (32 + s) with
    # s = ceil(log2 d), m = ceil(2^(32+s) / d), for n < 2^31. Check the
    # identity (and that n * m fits in 64 bits) at every quotient boundary
    # for every row width up to 8192 vectors.
    for d in range(1, 8193):
        s = (d - 1).bit_length()
        m = -(-(1 << (32 + s)) // d)
        assert m < (1 << 33)
        qmax = ((1 << 31) - 1) // d
        for q in {0, 1, 2, qmax // 3, qmax // 2, qmax - 1, qmax}:
            for n in (q * d - 1, q * d, q * d + d - 1):
                if 0 <= n < (1 << 31):
                    assert n * m < (1 << 64)
                    assert (n * m) >> (32 + s) == n // d, (d, n)


def test_dispatch_quant_validation(B):
    assert B.mep_quant_msg_bytes(7168) == 7680
    assert B.mep_quant_msg_bytes(100) == 512
    assert B.mep_quant_msg_bytes(0) == 0
    f = B.mep_dispatch_quant
    assert f(0, 2, 64, None, None, 0, None, None, 0, 512, None, None) == B.MEP_OK
    assert f(4, 2, 64, 16, None, 0, None, 16, 8, 512, None, None) == B.MEP_ERR_NULLPTR
    assert f(4, 2, 64, 16, None, 0, None, 16, 8, 64, 16, None) == B.MEP_ERR_SHAPE     # < H+4
    assert f(4, 2, 64, 16, None, 0, None, 16, 8, 520, 16, None) == B.MEP_ERR_SHAPE    # % 16
    assert f(4, 2, 16392, 16, None, 0, None, 16, 8, 16896, 16, None) == B.MEP_ERR_SHAPE
    assert f(4, 2, 64, 16, 16, 3, None, 16, 8, 512, 16, None) == B.MEP_ERR_PARAM     # no experts
    assert f(4, 2, 64, 16, 16, 0, 16, 16, 8, 512, 16, None) == B.MEP_ERR_PARAM       # E < 1
    assert f(4, 2, 64, 8, None, 0, None, 16, 8, 512, 16, None) == B.MEP_ERR_SHAPE    # unaligned x


def test_group_quant_validation(B):
    f = B.mep_group_quant
    assert f(0, 64, 512, None, 0, None, None, None, None) == B.MEP_OK
    assert f(4, 64, 512, 16, 4, 16, None, 16, None) == B.MEP_ERR_NULLPTR
    assert f(4, 64, 64, 16, 4, 16, 16, 16, None) == B.MEP_ERR_SHAPE      # msg too small
    assert f(4, 60, 512, 16, 4, 16, 16, 16, None) == B.MEP_ERR_SHAPE     # H % 8
    assert f(4, 64, 512, 16, 4, 16, 12, 16, None) == B.MEP_ERR_SHAPE     # x_q not 8-aligned


def test_plan_weight_rows_validation(B):
    f = B.mep_plan_weight_rows
    assert f(0, 8, 2, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert f(4, 2000, 2, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert f(4, 8, -1, 16, 16, 16, None) == B.MEP_ERR_PARAM
    assert f(4, 8, 2, None, 16, 16, None) == B.MEP_ERR_NULLPTR


def test_plan_dedup_validation(B):
    assert B.mep_plan_dedup_workspace_size(65, 10, 2) == 0
    n = B.mep_plan_dedup_workspace_size(8, 4096, 8)
    assert n > 0 and n % 256 == 0
    f = B.mep_plan_dedup
    assert f(8, 16, 2, 8, 16, 16, 256, n, 16, 16, 16, 16, None) == B.MEP_ERR_PARAM   # my_rank
    assert f(65, 16, 2, 0, 16, 16, 256, n, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE
    assert f(8, 16, 2, 0, None, 16, 256, n, 16, 16, 16, 16, None) == B.MEP_ERR_NULLPTR
    assert f(8, 16, 2, 0, 16, 16, 256, 8, 16, 16, 16, 16, None) == B.MEP_ERR_PARAM   # small ws
    m = B.mep_plan_dedup_workspace_size(8, 16, 2)
    assert f(8, 16, 2, 0, 16, 16, 16, m, 16, 16, 16, 16, None) == B.MEP_ERR_SHAPE    # ws align


def test_c_consumer_builds(B):
    # the plain C consumer of the ABI compiles and links against the library
    # and the oracle with gcc (it runs in the GPU suite)
    import __graft_entry__ as g
    import oracle
    oracle.build()
    assert os.path.exists(g.build_c_abi_check())


def test_plan_noalloc_validation(B):
    # argument errors are found on the host before the static array is
    # looked up or anything is enqueued; sizes whose workspace exceeds the
    # array are refused
    f = B.mep_plan_noalloc
    outs = [16] * 12
    assert f(2, 4, 8, 2, 0, None, *outs, None) == B.MEP_ERR_NULLPTR
    assert f(2, 4, 8, 2, 0, 16, *([None] + outs[1:]), None) == B.MEP_ERR_NULLPTR
    assert f(2, 4, 8, 2, 2, 16, *outs, None) == B.MEP_ERR_PARAM          # my_rank == R
    assert f(2, 4, 8, 5, 0, 16, *outs, None) == B.MEP_ERR_PARAM          # K > E
    assert f(0, 4, 8, 2, 0, 16, *outs, None) == B.MEP_ERR_SHAPE
    o = list(outs)
    o[2] = None                                                        # route_dest alone
    assert f(2, 4, 8, 2, 0, 16, *o, None) == B.MEP_ERR_PARAM
    big = (1024, 1024, 64, 2)
    assert B.mep_plan_workspace_size(*big) > B.MEP_PLAN_NOALLOC_SCRATCH_BYTES
    assert f(*big, 0, 16, *outs, None) == B.MEP_ERR_SHAPE
    # the workloads of the benchmark fit
    for R, E, S, K in [(8, 256, 4096, 8), (64, 256, 8192, 8), (8, 384, 8192, 8)]:
        assert 0 < B.mep_plan_workspace_size(R, E, S, K) <= B.MEP_PLAN_NOALLOC_SCRATCH_BYTES
