"""The C-ABI library loads, exports every declared symbol, and its host-only
validator returns the documented status for each error (no GPU needed)."""

import ctypes
import os
import re

import pytest

import tiled_exact_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built (python -m tiled_exact_attention_fa_amd.build)")
    return fa.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(fa_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header():
    # sizes follow from the field lists of include/fa.h on LP64
    assert ctypes.sizeof(fa.FaFwdParams) == 5 * 8 + 8 * 4 + 4 * 24 + 16 + 4 * 5 + 4
    assert ctypes.sizeof(fa.FaDecodeParams) == 8 * 8 + 6 * 4 + 16 + 24 + 16 + 16 + 16 + 8 + 8 + 8


def good_fwd():
    p = fa.FaFwdParams()
    p.q = p.k = p.v = p.o = 0x10000
    p.lse = 0
    p.in_dtype = p.out_dtype = fa.FA_BF16
    p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.d = 2, 8, 2, 100, 100, 128
    for name in ("q_strides", "k_strides", "v_strides", "o_strides"):
        setattr(p, name, fa.I64x3(8 * 100 * 128, 100 * 128, 128))
    p.softmax_scale = 128 ** -0.5
    return p


def test_fwd_validator_accepts_good_params(lib):
    assert fa.fa_check_fwd_params(good_fwd()) == fa.FA_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "q", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "Hkv", 3), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "B", -1), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "d", 96), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "out_dtype", fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "in_dtype", fa.FA_INT8), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "softmax_scale", 0.0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "softmax_scale", float("nan")), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "k", 0x10008), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "v_strides", fa.I64x3(1, 1, 132)), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "o_strides", fa.I64x3(0, 0, 64)), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "k_strides", fa.I64x3(0, 0, 1 << 24)), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "lse", 0x10002), fa.FA_ERR_ALIGNMENT),
])
def test_fwd_validator_errors(lib, mutate, status):
    p = good_fwd()
    mutate(p)
    assert fa.fa_check_fwd_params(p) == status
    assert fa.fa_last_error() != ""


def test_fwd_fp8_needs_positive_descales(lib):
    p = good_fwd()
    p.in_dtype = fa.FA_FP8_E4M3
    for name in ("q_strides", "k_strides", "v_strides"):
        setattr(p, name, fa.I64x3(8 * 100 * 128, 100 * 128, 128))
    p.q_descale = p.k_descale = p.v_descale = 1.0
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p.v_descale = 0.0
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_INVALID_ARG


def test_fwd_empty_problem_is_ok(lib):
    p = good_fwd()
    p.Sq = 0
    p.q = p.o = 0
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p = good_fwd()
    p.Sk = 0
    p.k = p.v = 0
    assert fa.fa_check_fwd_params(p) == fa.FA_OK


def good_decode():
    p = fa.FaDecodeParams()
    p.q = p.k_cache = p.v_cache = p.k_scale = p.v_scale = p.o = 0x20000
    p.B, p.Hq, p.Hkv, p.L, p.d, p.num_splits = 4, 32, 8, 1000, 128, 16
    p.q_strides = fa.I64x2(32 * 128, 128)
    p.kv_strides = fa.I64x3(8 * 1000 * 128, 1000 * 128, 128)
    p.scale_strides = fa.I64x2(8 * 1000, 1000)
    p.o_strides = fa.I64x2(32 * 128, 128)
    p.softmax_scale = 128 ** -0.5
    p.workspace = 0x40000
    p.workspace_bytes = fa.fa_decode_workspace_size(4, 32, 128, 16)
    return p


def test_decode_workspace_size(lib):
    # 16 splits x 64 batch x 32 heads x (128 floats + 1 float), each part 256-byte rounded
    rows = 16 * 64 * 32
    assert fa.fa_decode_workspace_size(64, 32, 128, 16) == rows * 128 * 4 + rows * 4
    assert fa.fa_decode_workspace_size(1, 1, 128, 1) == 512 + 256
    assert fa.fa_decode_workspace_size(1, 1, 128, 0) == 0
    assert fa.fa_decode_workspace_size(1, 1, 128, 65) == 0


def test_decode_validator(lib):
    assert fa.fa_check_decode_params(good_decode()) == fa.FA_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "k_cache", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "Hkv", 5), fa.FA_ERR_INVALID_ARG),
    (lambda p: (setattr(p, "Hkv", 1)), fa.FA_ERR_UNSUPPORTED),  # 32 heads per cache head
    (lambda p: setattr(p, "d", 64), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "num_splits", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "num_splits", 65), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "kv_format", 7), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "workspace_bytes", 100), fa.FA_ERR_WORKSPACE),
    (lambda p: setattr(p, "workspace", 0), fa.FA_ERR_WORKSPACE),
    (lambda p: setattr(p, "v_scale", 0x20001), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "scale_strides", fa.I64x2(8 * 1000, -1)), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "softmax_scale", -1.0), fa.FA_ERR_INVALID_ARG),
])
def test_decode_validator_errors(lib, mutate, status):
    p = good_decode()
    mutate(p)
    assert fa.fa_check_decode_params(p) == status


def test_status_strings(lib):
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(-4) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_string(-99) == "FA_ERR_UNKNOWN"
    fa.fa_check_fwd_params(good_fwd())
    assert fa.fa_last_error() == ""
