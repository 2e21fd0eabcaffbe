"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host (status codes and
messages) before any device call."""
import ctypes as C
import os
import re

import pytest

import sharded_gemm_alltosharded_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shardgemm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sg_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sg.LIB_PATH):
        pytest.skip("library not built")
    return sg.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for must in ("sg_shard_linear", "sg_shard_quantized_linear", "sg_all_to_sharded", "sg_sharded_to_all",
                 "sg_summa_matmul", "sg_layer_free", "sg_last_error"):
        assert must in names


def test_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def _err(L):
    return L.sg_last_error().decode()


def _shard(L, out_dims, in_dims, mode, segments, P, weight=1, dtype=sg.BF16):
    h = C.c_void_p()
    w = C.c_void_p(0x1000) if weight else None  # never dereferenced: validation fails first
    return L.sg_shard_linear(w, dtype, out_dims, in_dims, None, mode, segments, P, None, C.byref(h)), h


def test_output_not_divisible(L):
    rc, h = _shard(L, 3, 2, sg.ALL_TO_SHARDED, 1, 2)
    assert rc == sg.ERR_NOT_DIVISIBLE and h.value is None
    assert _err(L) == "Cannot shard the output of size 3 across 2 devices."


def test_input_not_divisible(L):
    rc, _ = _shard(L, 4, 6, sg.SHARDED_TO_ALL, 1, 4)
    assert rc == sg.ERR_NOT_DIVISIBLE
    assert "input of size 6 across 4" in _err(L)


def test_segments_rules(L):
    assert _shard(L, 10, 4, sg.ALL_TO_SHARDED, 3, 1)[0] == sg.ERR_NOT_DIVISIBLE  # 10 % 3
    assert "output of size 10 into 3 segments" in _err(L)
    assert _shard(L, 12, 4, sg.ALL_TO_SHARDED, 2, 4)[0] == sg.ERR_NOT_DIVISIBLE  # (12/2) % 4
    assert "output of size 12 across 4 devices" in _err(L)
    assert _shard(L, 4, 12, sg.SHARDED_TO_ALL, 2, 4)[0] == sg.ERR_NOT_DIVISIBLE  # input side, (12/2) % 4
    assert "input of size 12 across 4 devices" in _err(L)


def test_bad_mode(L):
    rc, _ = _shard(L, 4, 4, 7, 1, 2)
    assert rc == sg.ERR_BAD_MODE
    assert "all-to-sharded" in _err(L) and "sharded-to-all" in _err(L)


def test_invalid_args(L):
    assert _shard(L, 4, 4, 0, 1, 2, weight=0)[0] == sg.ERR_INVALID_ARG
    assert _shard(L, 4, 4, 0, 0, 2)[0] == sg.ERR_INVALID_ARG
    assert _shard(L, 4, 4, 0, 1, 0)[0] == sg.ERR_INVALID_ARG
    assert _shard(L, 0, 4, 0, 1, 1)[0] == sg.ERR_INVALID_ARG
    assert _shard(L, 4, 4, 0, 1, 1, dtype=9)[0] == sg.ERR_INVALID_ARG
    assert L.sg_shard_linear(C.c_void_p(0x1000), sg.BF16, 4, 4, None, 0, 1, 1, None, None) == sg.ERR_INVALID_ARG


def test_quantized_rules(L):
    h = C.c_void_p()
    p = C.c_void_p(0x1000)
    args = dict(out=8, inn=128, gs=64, bits=4, act=sg.BF16, mode=0, S=1, P=2)

    def call(**kw):
        a = {**args, **kw}
        return L.sg_shard_quantized_linear(p, p, p, a["out"], a["inn"], a["gs"], a["bits"], a["act"], None,
                                           a["mode"], a["S"], a["P"], None, C.byref(h))

    assert call(gs=32) == sg.ERR_UNSUPPORTED
    assert call(bits=8) == sg.ERR_UNSUPPORTED
    assert call(act=sg.F32) == sg.ERR_INVALID_ARG
    assert call(out=7) == sg.ERR_NOT_DIVISIBLE
    assert call(mode=1, inn=128, P=4) == sg.ERR_NOT_DIVISIBLE  # 32 inputs per rank < one group
    assert "straddle" in _err(L)
    assert call(mode=5) == sg.ERR_BAD_MODE


def test_forward_calls_validate_first(L):
    assert L.sg_all_to_sharded(None, None, 4, None, 0, 0, sg.BF16, None) == sg.ERR_INVALID_ARG
    assert L.sg_sharded_to_all(None, None, 4, None, sg.BF16, None, 0, None) == sg.ERR_INVALID_ARG
    assert L.sg_sharded_to_all_workspace(None, 4) == 0
    assert L.sg_all_to_sharded_ex(None, None, 0, 4, None, 0, 0, sg.BF16, None) == sg.ERR_INVALID_ARG
    h = C.c_void_p()
    assert L.sg_shard_mxfp8_linear(None, None, 64, 64, sg.BF16, None, 0, 1, 1, None, C.byref(h)) == sg.ERR_INVALID_ARG
    assert L.sg_sharded_to_all_ex(None, None, 4, None, 0, sg.BF16, None, 0, None) == sg.ERR_INVALID_ARG
    assert L.sg_layer_info(None, None, None, None, None, None, None, None) == sg.ERR_INVALID_ARG
    assert L.sg_layer_copy_shard(None, 0, 0, None, 0, None) == sg.ERR_INVALID_ARG
    L.sg_layer_free(None)  # ignored
    assert L.sg_mlp(None, None, None, 4, None, sg.BF16, None, 0, None) == sg.ERR_INVALID_ARG
    assert "NULL" in _err(L)
    assert L.sg_mlp_workspace(None, None, 4) == 0


def test_summa_rules(L):
    X = C.c_void_p(0x1000)
    assert L.sg_summa_matmul(X, X, sg.BF16, 8, 8, 8, 0, X, 0, 1, None, 0, None) == sg.ERR_NOT_DIVISIBLE  # q < 1
    assert L.sg_summa_matmul(X, X, sg.BF16, 6, 8, 8, 4, X, 0, 1, None, 0, None) == sg.ERR_NOT_DIVISIBLE
    assert L.sg_summa_matmul(X, X, sg.BF16, 8, 6, 8, 4, X, 0, 1, None, 0, None) == sg.ERR_NOT_DIVISIBLE
    assert L.sg_summa_matmul(X, X, 7, 8, 8, 8, 2, X, 0, 1, None, 0, None) == sg.ERR_INVALID_ARG
    assert L.sg_summa_matmul(X, X, sg.BF16, 8, 8, 8, 2, X, 2, 1, None, 0, None) == sg.ERR_INVALID_ARG
    # empty output: nothing to do, no device work
    assert L.sg_summa_matmul(None, None, sg.BF16, 0, 8, 8, 2, None, 0, 1, None, 0, None) == sg.OK
    # a workspace below the required size is rejected before any device work
    assert L.sg_summa_matmul(None, None, sg.BF16, 0, 64, 16, 2, None, 0, 1, X, 100, None) == sg.ERR_WORKSPACE


def test_summa_workspace_sizes(L):
    # the transposed fragment-major copy of A: K N 16-bit elements
    assert L.sg_summa_workspace(sg.BF16, 8192, 8192, 4) == 8192 * 8192 * 2
    assert L.sg_summa_workspace(sg.F16, 64, 48, 2) == 64 * 48 * 2
    # no copy where the fragment layout does not apply
    assert L.sg_summa_workspace(sg.F32, 64, 64, 2) == 0       # no fp32 MFMA path
    assert L.sg_summa_workspace(sg.BF16, 64, 40, 2) == 0      # N % 16
    assert L.sg_summa_workspace(sg.BF16, 96, 64, 2) == 0      # K / q = 48, not a multiple of 32
    assert L.sg_summa_workspace(sg.BF16, 64, 64, 3) == 0      # q does not divide K
    assert L.sg_summa_workspace(sg.BF16, 64, 64, 0) == 0


def test_binding_maps_sharding_names():
    assert sg._mode("all-to-sharded") == sg.ALL_TO_SHARDED
    assert sg._mode("sharded-to-all") == sg.SHARDED_TO_ALL
    assert sg._mode("column") == -1  # rejected by the library as a bad mode
