"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-side checks return the documented status codes
before any HIP call (run with -m "not gpu")."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_act.h")
LIB = os.path.join(ROOT, "sparse_input_gemv_amd", "libsparse_act.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s+(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def sa():
    import sparse_input_gemv_amd as m
    return m.lib()


# Plausible, aligned addresses that are never dereferenced: every call below
# fails a host check first (or is an empty call that returns before HIP).
P = 1 << 20


def test_every_declared_symbol_is_exported(sa):
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(sa, n), n
    # the hot path's six calls and its workspace query, by the contract's names
    for n in ("act_sparsify_threshold", "act_sparsify_topk", "act_sparsify_nm", "sparse_gemv",
              "masked_swiglu_down", "nm_act_spmm", "sparse_gemv_workspace_bytes",
              "act_calibrate_threshold", "sa_workspace_zero_bytes"):
        assert n in names


def test_status_strings(sa):
    assert sa.sa_status_string(SA_OK) == b"SA_OK"
    assert sa.sa_status_string(SA_ERR_WORKSPACE) == b"SA_ERR_WORKSPACE"
    assert sa.sa_status_string(99) == b"SA_ERR_UNKNOWN"
    assert sa.sa_version() == 100


def test_threshold_checks(sa):
    f = sa.act_sparsify_threshold
    assert f(None, 1, 16, 0.5, None, P, P, P, 16, None) == SA_ERR_INVALID_ARG
    assert b"x is NULL" in sa.sa_last_error()
    assert f(P, 1, 0, 0.5, None, P, P, P, 16, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 16, 0.5, None, P, P, P, 15, None) == SA_ERR_INVALID_ARG  # cap < d
    assert f(P, 1, 16, -1.0, None, P, P, P, 16, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 16, float("nan"), None, P, P, P, 16, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 70000, 0.5, None, P, P, P, 70000, None) == SA_ERR_UNSUPPORTED
    assert f(P + 1, 1, 16, 0.5, None, P, P, P, 16, None) == SA_ERR_INVALID_ARG  # misaligned
    assert f(P, 0, 16, 0.5, None, P, P, P, 16, None) == SA_OK  # empty call
    assert sa.sa_last_error() == b""


def test_topk_checks(sa):
    f = sa.act_sparsify_topk
    assert f(P, 1, 16, 17, None, P, P, P, 17, None) == SA_ERR_INVALID_ARG  # k > d
    assert f(P, 1, 16, -1, None, P, P, P, 16, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 16, 8, None, P, P, P, 7, None) == SA_ERR_INVALID_ARG  # cap < k
    assert f(P, 1, 16, 8, None, None, P, P, 8, None) == SA_ERR_INVALID_ARG
    assert f(P, 0, 16, 8, None, P, P, P, 8, None) == SA_OK


def test_topk_cutoff_checks(sa):
    f = sa.act_topk_cutoff  # (x, rows, d, k, cut, stream)
    assert f(P, 1, 16, 17, P, None) == SA_ERR_INVALID_ARG  # k > d
    assert f(P, 1, 16, -1, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 16, 8, None, None) == SA_ERR_INVALID_ARG  # no output
    assert f(P, 1, 16, 8, P + 4, None) == SA_ERR_INVALID_ARG  # cut not 8-byte aligned
    assert f(P + 1, 1, 16, 8, P, None) == SA_ERR_INVALID_ARG  # x misaligned
    assert f(P, 1, 70000, 8, P, None) == SA_ERR_UNSUPPORTED  # d > 65536
    assert f(P, 0, 16, 8, None, None) == SA_OK  # empty call


def test_sparse_gemv_topk_checks(sa):
    # (wt, d_out, d_in, x, batch, k, y, ws, ws_bytes, stream)
    f = sa.sparse_gemv_topk
    need = sa.sparse_gemv_workspace_bytes(4096, 11008, 1)
    ok = [P, 4096, 11008, P, 1, 5504, P, P, need, None]
    args = list(ok)
    args[5] = 11009  # k > d_in
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[5] = -1
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[3] = None  # x
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[8] = need - 1
    assert f(*args) == SA_ERR_WORKSPACE
    args = list(ok)
    args[2] = 70000  # the select takes rows of at most 65536
    args[8] = sa.sparse_gemv_workspace_bytes(4096, 70000, 1)
    args[5] = 100
    assert f(*args) == SA_ERR_UNSUPPORTED
    args = list(ok)
    args[4] = 0  # empty batch, arguments still checked
    args[5] = 11009
    assert f(*args) == SA_ERR_INVALID_ARG
    args[5] = 10
    assert f(*args) == SA_OK


def test_nm_checks(sa):
    f = sa.act_sparsify_nm
    assert f(P, 1, 64, 2, 6, P, P, None) == SA_ERR_INVALID_ARG  # m not supported
    assert f(P, 1, 64, 0, 4, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 64, 5, 4, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 1, 48, 2, 4, P, P, None) == SA_ERR_INVALID_ARG  # d % 32
    assert f(P + 8, 1, 64, 2, 4, P, P, None) == SA_ERR_INVALID_ARG  # x not 16-B aligned
    assert f(P, 0, 64, 2, 4, P, P, None) == SA_OK


def test_nm_shared_checks(sa):
    f = sa.act_sparsify_nm_shared  # (x, rows, d, n, m, tt, mask, val, stream)
    assert f(P, 4, 64, 2, 4, 0, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 64, 2, 4, 257, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 64, 2, 6, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 64, 5, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 64, 0, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 48, 2, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(None, 4, 64, 2, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P + 8, 4, 64, 2, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 4, 64, 2, 4, 32, P + 2, P, None) == SA_ERR_INVALID_ARG
    assert f(P, -1, 64, 2, 4, 32, P, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 0, 64, 2, 4, 32, P, P, None) == SA_OK  # nothing to do

    g = sa.nm_shared_spmm  # (xval, mask, T, d_in, n, m, tt, wt, d_out, y, ws, ws_bytes, stream)
    assert g(P, P, 4, 64, 2, 4, 0, P, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 4, 64, 2, 4, 300, P, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 4, 64, 2, 5, 32, P, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 4, 40, 2, 4, 32, P, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 4, 64, 2, 4, 32, P, 60, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 4, 64, 2, 4, 32, P + 8, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert g(P, None, 4, 64, 2, 4, 32, P, 64, P, None, 0, None) == SA_ERR_INVALID_ARG
    # the expansion path needs a workspace: refused on the host, before any launch
    assert g(P, P, 4, 64, 3, 4, 32, P, 64, P, None, 0, None) == SA_ERR_WORKSPACE
    assert g(P, P, 4, 64, 3, 4, 32, P, 64, P, P, 100, None) == SA_ERR_WORKSPACE
    assert g(P, P, 4, 64, 8, 16, 16, P, 64, P, None, 0, None) == SA_ERR_WORKSPACE
    assert g(P, P, 4, 64, 3, 4, 32, P, 64, P, P + 8, 4 * 64 * 2, None) == SA_ERR_INVALID_ARG
    assert g(P, P, 0, 64, 2, 4, 32, P, 64, P, None, 0, None) == SA_OK  # nothing to do

    ws = sa.sa_nm_shared_spmm_workspace_bytes  # (T, d_in, n, m, tt)
    assert ws(100, 1024, 8, 16, 32) == 0
    assert ws(100, 1024, 4, 16, 64) == 0
    assert ws(100, 1024, 8, 16, 16) == 100 * 1024 * 2
    assert ws(100, 1056, 8, 16, 32) == 100 * 1056 * 2  # d_in not a multiple of the K step
    assert ws(100, 1024, 3, 4, 32) == 100 * 1024 * 2
    assert ws(100, 1024, 1, 8, 32) == 0                # m / n = 8: 32-row-tile gather
    assert ws(100, 1024, 32, 32, 32) == 0               # m / n = 1: 32-row-tile gather
    assert ws(100, 1024, 1, 8, 48) == 100 * 1024 * 2    # tiles not a multiple of 32 rows
    assert ws(100, 40000, 8, 16, 32) == 0  # past the 32-row gather's mask copy: per-block gather
    assert ws(100, 1024, 1, 8, 128) == 0               # whole-tile gather
    assert ws(100, 1024, 3, 4, 128) == 100 * 1024 * 2   # n does not divide 32
    assert ws(10, 65536, 1, 8, 128) == 10 * 65536 * 2   # mask row beyond the LDS copy
    assert ws(0, 1024, 8, 16, 32) == 0
    assert ws(100, 1024, 8, 16, 0) == 0


def test_calibrate_checks(sa):
    f = sa.act_calibrate_threshold
    assert f(P, 0, 0.5, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 10, 1.5, P, None) == SA_ERR_INVALID_ARG
    assert f(None, 10, 0.5, P, None) == SA_ERR_INVALID_ARG


def test_workspace_size(sa):
    a = sa.sa_workspace_bytes(4096, 11008, 1)
    b = sa.sa_workspace_bytes(4096, 11008, 8)
    assert 0 < a < b
    assert a % 256 == 0 or a > 0
    assert sa.sa_workspace_bytes(0, 10, 1) == 0
    # the zero-once hand-off counters lead every workspace
    assert sa.sa_workspace_bytes(8, 1, 1) > 1 << 20
    # the contract's name is the same function
    for shape in ((4096, 11008, 1), (4096, 11008, 8), (22016, 4096, 2), (8, 1, 1), (0, 10, 1)):
        assert sa.sparse_gemv_workspace_bytes(*shape) == sa.sa_workspace_bytes(*shape)
    assert sa.sa_workspace_zero_bytes(4096, 11008, 1) == 1 << 20
    assert sa.sa_workspace_zero_bytes(4096, 11008, 1) < sa.sa_workspace_bytes(4096, 11008, 1)


def test_gemv_checks(sa):
    need = sa.sa_workspace_bytes(4096, 11008, 1)
    f = sa.sparse_gemv
    assert f(P, 4100, 11008, P, P, P, 1, 11008, P, P, need, None) == SA_ERR_INVALID_ARG  # d_out%8
    assert f(P, 4096, 11008, P, P, P, 9, 11008, P, P, need * 9, None) == SA_ERR_INVALID_ARG
    assert f(P, 4096, 11008, P, P, P, 1, 11008, P, P, need - 1, None) == SA_ERR_WORKSPACE
    assert f(P, 4096, 11008, P, P, P, 1, 11008, P, None, 0, None) == SA_ERR_WORKSPACE
    assert f(P, 4096, 11008, None, P, P, 1, 11008, P, P, need, None) == SA_ERR_INVALID_ARG
    assert f(P + 2, 4096, 11008, P, P, P, 1, 11008, P, P, need, None) == SA_ERR_INVALID_ARG
    assert f(P, 4096, 11008, P, P, P, 0, 11008, P, P, need, None) == SA_OK  # empty batch
    g = sa.sparse_gemv_threshold
    assert g(P, 4096, 11008, P, 1, -0.5, P, P, need, None) == SA_ERR_INVALID_ARG
    assert g(P, 4096, 11008, None, 1, 0.5, P, P, need, None) == SA_ERR_INVALID_ARG
    h = sa.masked_gemv
    assert h(P, 4096, 11008, P, None, 1, P, P, need, None) == SA_ERR_INVALID_ARG
    d = sa.dense_gemv
    assert d(P, 4096, 11008, None, 1, P, P, need, None) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemv_tuning(99, 0, 0) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemv_tuning(-1, 0, 4) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemv_tuning(-1, -1, 0) == SA_ERR_INVALID_ARG
    for handoff in (1, 2, 3, 0):
        assert sa.sa_set_gemv_tuning(-1, 0, handoff) == SA_OK
    assert sa.sa_set_gemm_tuning(64, 0, 0) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemm_tuning(0, 4, 0) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemm_tuning(128, 3, 0) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemm_tuning(0, -1, 0) == SA_ERR_INVALID_ARG
    for stages in (1, 2, 7, -1):
        assert sa.sa_set_gemm_tuning(0, 0, stages) == SA_ERR_INVALID_ARG
    for rows, engine, stages in ((128, 1, 0), (256, 2, 4), (128, 2, 6), (0, 3, 0), (256, 3, 6),
                                 (0, 0, 0)):
        assert sa.sa_set_gemm_tuning(rows, engine, stages) == SA_OK


def test_scored_and_corrected_checks(sa):
    f = sa.act_sparsify_scored
    ok = [P, 1, 64, None, None, 0, 0, 0.5, P, P, P, P, 64, None, None]  # never called as is
    args = list(ok)
    args[7] = -1.0
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[5], args[6] = 2, 6  # m not supported
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[2], args[5], args[6] = 60, 2, 8  # d % m
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[5], args[6], args[12] = 8, 16, 31  # cap < d*n/m = 32
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[4] = P + 4  # colnorm not 8-byte aligned
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[1] = 0
    assert f(*args) == SA_OK
    g = sa.sparse_gemv_corrected
    need = sa.sa_workspace_bytes(4096, 11008, 1)
    okg = [P, 4096, 11008, P, P, P, 1, 11008, None, None, P, P, need, None]
    args = list(okg)
    args[8] = P + 2  # alpha misaligned
    assert g(*args) == SA_ERR_INVALID_ARG
    args = list(okg)
    args[12] = need - 1
    assert g(*args) == SA_ERR_WORKSPACE
    args = list(okg)
    args[6] = 0
    assert g(*args) == SA_OK


def test_scored_gemv_checks(sa):
    need = sa.sa_workspace_bytes(4096, 11008, 1)
    f = sa.sparse_gemv_scored
    ok = [P, 4096, 11008, P, None, None, 0.5, 1, None, P, P, need, None]  # never called as is
    args = list(ok)
    args[6] = -0.5
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[6] = float("nan")
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[5] = P + 4  # colnorm not 8-byte aligned
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[11] = need - 1
    assert f(*args) == SA_ERR_WORKSPACE
    args = list(ok)
    args[3] = None
    assert f(*args) == SA_ERR_INVALID_ARG


def test_scored_nm_gemv_checks(sa):
    need = sa.sa_workspace_bytes(4096, 11008, 1)
    f = sa.sparse_gemv_scored_nm
    ok = [P, 4096, 11008, P, None, None, 8, 16, 1, None, P, P, need, None]  # never called as is
    for n, m in [(0, 16), (17, 16), (2, 6), (2, 64), (1, 2), (-1, 4)]:
        args = list(ok)
        args[6], args[7] = n, m
        assert f(*args) == SA_ERR_INVALID_ARG, (n, m)
    args = list(ok)
    args[2] = 11000  # not a multiple of m = 16
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[5] = P + 4  # colnorm not 8-byte aligned
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[12] = need - 1
    assert f(*args) == SA_ERR_WORKSPACE
    args = list(ok)
    args[3] = None
    assert f(*args) == SA_ERR_INVALID_ARG


def test_rana_adapter_checks(sa):
    # B is row-major and needs no workspace: only the second GEMV's counts
    need = sa.sa_workspace_bytes(11008, 2048, 1)
    f = sa.rana_adapter_gemv
    ok = [P, 2048, 4096, P, 11008, P, 1, 0.5, P, P, P, need, None]
    args = list(ok)
    args[1] = 0  # r
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[0] = None  # b
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[0] = P + 1  # b misaligned
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[4] = 11004  # d_out % 8
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[7] = -1.0
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[11] = need - 1
    assert f(*args) == SA_ERR_WORKSPACE
    args = list(ok)
    args[5] = None  # x
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[8] = P + 1  # v misaligned
    assert f(*args) == SA_ERR_INVALID_ARG
    args = list(ok)
    args[6] = 0  # empty batch: nothing to do
    assert f(*args) == SA_OK


def test_swiglu_checks(sa):
    need = sa.sa_workspace_bytes(4096, 14336, 1)
    f = sa.masked_swiglu_down
    args = [P, P, P, None, 14336, 4096, 0.5, 1, P, None, None, P, need, None]
    assert f(*args) == SA_ERR_INVALID_ARG  # RaNA needs colnorm
    args[7] = 2
    assert f(*args) == SA_ERR_INVALID_ARG  # unknown mode
    args[7] = 0
    args[6] = float("inf")
    assert f(*args) == SA_ERR_INVALID_ARG


def test_matmul_checks(sa):
    f = sa.nm_act_spmm
    assert f(P, P, 16, 1000, 2, 4, P, 1024, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert f(P, P, 16, 1024, 3, 2, P, 1024, P, None, 0, None) == SA_ERR_INVALID_ARG
    assert f(P, P, 0, 1024, 2, 4, P, 1024, P, None, 0, None) == SA_OK
    need = sa.sa_nm_spmm_workspace_bytes(16, 1024, 8, 16)
    assert need == 16 * 1024 * 2
    assert sa.sa_nm_spmm_workspace_bytes(16, 1024, 2, 4) == 0  # 2:4 needs none
    assert sa.sa_nm_spmm_workspace_bytes(16, 1024, 5, 4) == 0  # invalid pattern
    assert f(P, P, 16, 1024, 8, 16, P, 1024, P, P, need - 1, None) == SA_ERR_WORKSPACE
    assert f(P, P, 16, 1024, 8, 16, P, 1024, P, P + 8, need, None) == SA_ERR_INVALID_ARG
    g = sa.dense_gemm
    assert g(P, 16, 1020, P, 1024, P, None) == SA_ERR_INVALID_ARG
    assert g(P, 0, 1024, P, 1024, P, None) == SA_OK


def test_read_stream_checks(sa):
    f = sa.sa_read_stream
    assert f(None, 16, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 0, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 24, P, None) == SA_ERR_INVALID_ARG
    assert f(P + 8, 16, P, None) == SA_ERR_INVALID_ARG
    assert f(P, 16, None, None) == SA_ERR_INVALID_ARG


def test_tiling_info(sa):
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert sa.sa_gemv_tiling_info(0, ctypes.addressof(a), ctypes.addressof(b),
                                  ctypes.addressof(c)) == SA_OK
    assert (a.value, b.value, c.value) == (128, 256, 8)
    assert sa.sa_gemv_tiling_info(8, ctypes.addressof(a), None, None) == SA_OK and a.value == -16
    assert sa.sa_gemv_tiling_info(100, None, None, None) == SA_ERR_INVALID_ARG


def _plan(op, d_out, d_in, batch=1):
    """The decomposition on a 256-CU part with 8 resident workgroups per CU,
    computed on the host (no device involved)."""
    import sparse_input_gemv_amd as m
    return m.gemv_plan(op, d_out, d_in, batch, cus=256, resident=8)


def test_plan_headline_and_llama_shapes():
    # the headline: 32 tiles x 24 slices, one launch, partials in L2
    assert _plan("threshold", 4096, 11008) == {"kernel": "split-K", "tile_o": 128, "grid_o": 32,
                                               "slices": 24, "handoff": 3}
    assert _plan("dense", 4096, 11008)["slices"] == 32
    # 86 tiles are not a multiple of 8: at batch 1 the grid pads them to 88
    # (the padding workgroups exit at once), so the partials stay in L2
    p = _plan("threshold", 11008, 4096)
    assert (p["grid_o"], p["slices"], p["handoff"]) == (86, 8, 3)
    assert _plan("threshold", 11008, 2048)["handoff"] == 3  # the rank adapter's A
    assert _plan("threshold", 22016, 4096)["handoff"] == 3  # 172 tiles
    # fewer than 8 tiles are not padded: written through
    p = _plan("threshold", 640, 16384)
    assert (p["kernel"], p["grid_o"], p["handoff"]) == ("split-K", 5, 2)
    # balance: 4 slices (688 workgroups, <= 3 per CU) rather than 5 (860, <= 4)
    assert _plan("threshold", 22016, 4096)["slices"] == 4
    assert _plan("dense", 22016, 4096)["slices"] == 4
    assert _plan("dense", 12288, 4096)["slices"] == 8
    # batch 3..8: a second launch sums the partials
    assert _plan("threshold", 4096, 4096, 4)["handoff"] == 1
    assert _plan("masked", 4096, 4096, 8)["handoff"] == 1
    assert _plan("threshold", 4096, 4096, 2)["handoff"] == 3
    # batch 2: one launch only in L2 with at most 24 slices
    assert _plan("threshold", 4096, 11008, 2)["handoff"] == 3
    assert _plan("threshold", 11008, 4096, 2)["handoff"] == 1  # 86 tiles
    assert _plan("dense", 1024, 4096, 2)["handoff"] == 1  # 32 slices
    assert _plan("threshold", 11008, 4096, 1)["handoff"] == 3


def test_plan_small_weights():
    # tall-K small weights: split-K, one workgroup per CU, 64-wide tiles at batch 1
    p = _plan("threshold", 1024, 4096)
    assert (p["kernel"], p["tile_o"], p["grid_o"], p["slices"]) == ("split-K", 64, 16, 16)
    p = _plan("threshold", 1024, 4096, 2)
    assert (p["kernel"], p["tile_o"], p["grid_o"], p["slices"]) == ("split-K", 128, 8, 32)
    # slices of at least 128 rows
    p = _plan("dense", 256, 4096)
    assert p["kernel"] == "split-K" and 4096 // p["slices"] >= 128
    # full-K where its grid covers every CU or d_in is short
    assert _plan("threshold", 4096, 1024)["kernel"] == "full-K"
    assert _plan("list", 1024, 1024)["kernel"] == "full-K"
    assert _plan("dense", 4096, 512, 2)["kernel"] == "full-K"
    # not for batched lists or batch > 2
    assert _plan("list", 1024, 1024, 2)["kernel"] == "split-K"
    assert _plan("threshold", 4096, 1024, 4)["kernel"] == "split-K"
    # 8-16 MB: split-K, one workgroup per CU
    p = _plan("dense", 1024, 8192)
    assert (p["tile_o"], p["grid_o"] * p["slices"]) == (64, 256)


def test_plan_topk_forms(sa):
    import sparse_input_gemv_amd as m
    # batch 1, one launch, every workgroup selecting the cutoff: the split-K
    # plan of the threshold GEMV, also where the two-launch form would run
    # full-K
    assert _plan("topk", 11008, 4096) == _plan("threshold", 11008, 4096)
    assert _plan("topk", 4096, 1024)["kernel"] == "split-K"
    assert _plan("topk", 1024, 1024)["kernel"] == "split-K"
    try:
        m.set_gemv_test_hooks(2)  # the two-launch form
        assert _plan("topk", 4096, 1024)["kernel"] == "full-K"
        assert _plan("topk", 11008, 4096) == _plan("threshold", 11008, 4096)
    finally:
        m.set_gemv_test_hooks(0)
    # batch 2 and more: two launches, the threshold GEMV's plans
    assert _plan("topk", 4096, 4096, 2) == _plan("threshold", 4096, 4096, 2)
    assert _plan("topk", 1024, 1024, 2)["kernel"] == "full-K"
    assert _plan("topk", 4096, 1024, 4)["kernel"] == "split-K"


def _gplan(op, T, d_in, d_out, n=0, m=0):
    import sparse_input_gemv_amd as m_
    return m_.gemm_plan(op, T, d_in, d_out, n, m, cus=256)


def test_gemm_plan_engines(sa):
    import sparse_input_gemv_amd as m
    # 256 x 256 tiles only where their rounds over the CUs pay: 688 tiles of
    # 256 x 128 at 2048 x 4096 x 11008 (344 wide tiles would take 1.34 rounds)
    assert _gplan("dense", 2048, 4096, 11008) == {"engine": "pipelined", "tile_rows": 256,
                                                  "tile_cols": 128, "tiles": 688}
    assert _gplan("dense", 4096, 4096, 4096) == {"engine": "wide", "tile_rows": 256,
                                                 "tile_cols": 256, "tiles": 256}
    assert _gplan("dense", 2048, 4096, 13312)["tiles"] == 416  # wide, 1.6 rounds
    assert _gplan("dense", 2048, 4096, 13312)["engine"] == "wide"
    assert _gplan("dense", 4096, 4096, 11008)["engine"] == "wide"  # 688 wide tiles
    assert _gplan("dense", 3072, 4096, 11008)["engine"] == "pipelined"  # 516: just past 2 rounds
    # fewer 256-row tiles than CUs: 128-row tiles
    assert _gplan("dense", 4096, 1024, 1024) == {"engine": "pipelined", "tile_rows": 128,
                                                 "tile_cols": 128, "tiles": 256}
    # K not a multiple of 32: the staged-register engine
    assert _gplan("dense", 1000, 3000, 1032)["engine"] == "staged"
    # 2:4 on wide tiles once their rounds stay within 1.5x the tiles per CU,
    # else on 128-row pipelined tiles; other patterns on the dense engine's
    # choice for the expanded copy
    assert _gplan("nm", 2048, 4096, 11008, 2, 4) == {"engine": "wide", "tile_rows": 256,
                                                     "tile_cols": 256, "tiles": 344}
    assert _gplan("nm", 4096, 4096, 4096, 2, 4)["engine"] == "wide"
    assert _gplan("nm", 1024, 4096, 16384, 2, 4)["engine"] == "wide"  # 256: one whole round
    assert _gplan("nm", 2048, 4096, 4096, 2, 4) == {"engine": "pipelined", "tile_rows": 128,
                                                   "tile_cols": 128, "tiles": 512}
    assert _gplan("nm", 4096, 1024, 1024, 2, 4)["engine"] == "pipelined"
    assert _gplan("nm", 1024, 4096, 16640, 2, 4)["engine"] == "pipelined"  # 260: 2 rounds
    assert _gplan("nm", 4096, 4096, 4096, 8, 16)["engine"] == "wide"
    assert _gplan("nm", 2048, 4096, 11008, 16, 32)["engine"] == "pipelined"
    try:
        m.set_gemm_tuning(0, 3, 0)
        assert _gplan("dense", 2048, 4096, 11008)["engine"] == "wide"
        assert _gplan("nm", 2048, 4096, 11008, 2, 4) == {"engine": "wide", "tile_rows": 256,
                                                         "tile_cols": 256, "tiles": 344}
        m.set_gemm_tuning(0, 2, 0)
        assert _gplan("dense", 4096, 4096, 4096)["engine"] == "pipelined"
        m.set_gemm_tuning(128, 0, 0)
        assert _gplan("dense", 4096, 4096, 4096)["tile_rows"] == 128
        m.set_gemm_tuning(0, 1, 0)
        assert _gplan("dense", 4096, 4096, 4096)["engine"] == "staged"
    finally:
        m.set_gemm_tuning(0, 0, 0)


def test_gemm_plan_checks(sa):
    o = [ctypes.c_int() for _ in range(3)] + [ctypes.c_int64()]
    a = [ctypes.addressof(x) for x in o]
    assert sa.sa_gemm_plan(0, 2048, 4096, 11008, 0, 0, 256, *a) == SA_OK
    assert sa.sa_gemm_plan(1, 2048, 4096, 11008, 2, 4, 256, *a) == SA_OK
    assert sa.sa_gemm_plan(2, 2048, 4096, 11008, 0, 0, 256, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(1, 2048, 4096, 11008, 3, 5, 256, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(1, 2048, 4096, 11008, 5, 4, 256, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(1, 2048, 4100, 11008, 2, 4, 256, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(0, 0, 4096, 11008, 0, 0, 256, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(0, 2048, 4096, 11008, 0, 0, -1, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemm_plan(0, 2048, 4096, 11008, 0, 0, 256, None, *a[1:]) == SA_ERR_INVALID_ARG


def test_plan_follows_tuning(sa):
    import sparse_input_gemv_amd as m
    try:
        m.set_gemv_tuning(-1, 0, 2)
        assert _plan("threshold", 4096, 11008)["handoff"] == 2
        m.set_gemv_tuning(-1, 0, 1)
        assert _plan("threshold", 4096, 11008)["handoff"] == 1
        m.set_gemv_tuning(8, 0, 0)
        assert _plan("threshold", 4096, 11008)["kernel"] == "full-K"
        m.set_gemv_tuning(0, 1024, 0)
        p = _plan("threshold", 4096, 11008)
        assert p["grid_o"] * p["slices"] == 1024
    finally:
        m.set_gemv_tuning(-1, 0, 0)


def test_plan_checks(sa):
    o = [ctypes.c_int() for _ in range(5)]
    a = [ctypes.addressof(x) for x in o]
    assert sa.sa_gemv_plan(0, 4096, 11008, 1, 256, 8, *a) == SA_OK
    assert sa.sa_gemv_plan(5, 4096, 11008, 1, 256, 8, *a) == SA_ERR_INVALID_ARG  # unknown op
    assert sa.sa_gemv_plan(0, 0, 11008, 1, 256, 8, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemv_plan(0, 4096, 11008, 0, 256, 8, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemv_plan(0, 4096, 11008, 9, 256, 8, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemv_plan(0, 4096, 11008, 1, -1, 8, *a) == SA_ERR_INVALID_ARG
    assert sa.sa_gemv_plan(0, 4096, 11008, 1, 256, 8, None, *a[1:]) == SA_ERR_INVALID_ARG


def test_test_hook_checks(sa):
    assert sa.sa_set_gemv_test_hooks(4) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemv_test_hooks(-1) == SA_ERR_INVALID_ARG
    assert sa.sa_set_gemv_test_hooks(1) == SA_OK
    assert sa.sa_set_gemv_test_hooks(3) == SA_OK
    assert sa.sa_set_gemv_test_hooks(2) == SA_OK
    assert sa.sa_set_gemv_test_hooks(0) == SA_OK
