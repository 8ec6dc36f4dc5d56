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


STRUCTS = [("fa_fwd_params", fa.FaFwdParams), ("fa_decode_params", fa.FaDecodeParams),
           ("fa_kv_append_params", fa.FaKvAppendParams), ("fa_bwd_params", fa.FaBwdParams),
           ("fa_fp8_quant_params", fa.FaFp8QuantParams)]


def test_struct_layout_matches_header(tmp_path):
    # the C compiler's own sizeof / offsetof of every field of include/fa.h
    # against the ctypes mirrors
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fa.h"', "int main(void) {"]
    for cname, py in STRUCTS:
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess

    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(ln.split()[:2]): int(ln.split()[2]) for ln in out if ln.strip()}
    for cname, py in STRUCTS:
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


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


def test_fwd_sequence_stride_limit(lib):
    """Row offsets within a tile are formed in 32 bits for every row of the
    tile, also past the last key: a one-key K whose sequence stride exceeds
    8 MiB is refused although its extent is small; 8 MiB itself is accepted."""
    p = good_fwd()
    p.Sk = 1
    p.k_strides = fa.I64x3(0, 0, 1 << 22)  # 8 MiB of bf16 per row
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p.k_strides = fa.I64x3(0, 0, (1 << 22) + 8)
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_UNSUPPORTED
    assert "8 MiB" in fa.fa_last_error()


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
    (lambda p: setattr(p, "W", -1), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "W", 64), fa.FA_ERR_INVALID_ARG),  # window on, window pointers NULL
])
def test_decode_validator_errors(lib, mutate, status):
    p = good_decode()
    mutate(p)
    assert fa.fa_check_decode_params(p) == status


def good_window(p):
    p.k_recent = p.v_recent = 0x60000
    p.W = 64
    p.recent_strides = fa.I64x3(8 * 64 * 128, 64 * 128, 128)
    p.workspace_bytes = fa.fa_decode_workspace_size(4, 32, 128, 17)
    return p


def test_decode_fp8_format_and_window_accepted(lib):
    p = good_decode()
    p.kv_format = fa.FA_KV_FP8_E4M3_TOKHEAD_F16SCALE
    assert fa.fa_check_decode_params(p) == fa.FA_OK
    assert fa.fa_check_decode_params(good_window(good_decode())) == fa.FA_OK


@pytest.mark.parametrize("mutate,status", [
    # the window takes one more partial slot: the split-only size is too small
    (lambda p: setattr(p, "workspace_bytes", fa.fa_decode_workspace_size(4, 32, 128, 16)), fa.FA_ERR_WORKSPACE),
    (lambda p: setattr(p, "v_recent", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "k_recent", 0x60008), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "recent_strides", fa.I64x3(8 * 64 * 128, 64 * 128, 120)), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "recent_strides", fa.I64x3(8 * 64 * 128, 64 * 128, 132)), fa.FA_ERR_ALIGNMENT),
])
def test_decode_window_validator_errors(lib, mutate, status):
    p = good_window(good_decode())
    mutate(p)
    assert fa.fa_check_decode_params(p) == status


def good_append():
    p = fa.FaKvAppendParams()
    p.k_new = p.v_new = 0x10000
    p.k_cache = p.v_cache = 0x20000
    p.k_scale = p.v_scale = 0x30000
    p.in_dtype = fa.FA_BF16
    p.kv_format = fa.FA_KV_INT8_TOKHEAD_F16SCALE
    p.B, p.H, p.T, p.L, p.d = 4, 8, 16, 1000, 128
    p.new_strides = fa.I64x3(8 * 16 * 128, 16 * 128, 128)
    p.kv_strides = fa.I64x3(8 * 1000 * 128, 1000 * 128, 128)
    p.scale_strides = fa.I64x2(8 * 1000, 1000)
    return p


def test_append_validator(lib):
    assert fa.fa_check_kv_append_params(good_append()) == fa.FA_OK
    p = good_append()
    p.kv_format, p.in_dtype = fa.FA_KV_FP8_E4M3_TOKHEAD_F16SCALE, fa.FA_F16
    assert fa.fa_check_kv_append_params(p) == fa.FA_OK
    p = good_append()
    p.T = 0
    p.k_new = 0  # nothing to write: no tensor is looked at
    assert fa.fa_check_kv_append_params(p) == fa.FA_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "kv_format", 5), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "in_dtype", fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "d", 64), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "H", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "T", -1), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "v_new", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "k_cache", 0x20008), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "k_scale", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "v_scale", 0x30001), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "new_strides", fa.I64x3(8 * 16 * 128, 16 * 128, 120)), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "scale_strides", fa.I64x2(-1, 1000)), fa.FA_ERR_INVALID_ARG),
    (lambda p: (setattr(p, "B", 1 << 20), setattr(p, "H", 1 << 8), setattr(p, "T", 1 << 4)), fa.FA_ERR_UNSUPPORTED),
])
def test_append_validator_errors(lib, mutate, status):
    p = good_append()
    mutate(p)
    assert fa.fa_check_kv_append_params(p) == status


def test_status_strings(lib):
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(-4) == "FA_ERR_WORKSPACE"
    assert fa.fa_status_string(-99) == "FA_ERR_UNKNOWN"
    fa.fa_check_fwd_params(good_fwd())
    assert fa.fa_last_error() == ""


def good_bwd():
    p = fa.FaBwdParams()
    p.q = p.k = p.v = p.o = p.dout = p.dq = p.dk = p.dv = 0x10000
    p.lse = 0x20000
    p.dtype = fa.FA_BF16
    p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.d = 2, 8, 2, 100, 120, 128
    for name in ("q", "o", "do", "dq"):
        setattr(p, f"{name}_strides", fa.I64x3(8 * 100 * 128, 100 * 128, 128))
    for name in ("k", "v", "dk", "dv"):
        setattr(p, f"{name}_strides", fa.I64x3(2 * 120 * 128, 120 * 128, 128))
    p.lse_strides = fa.I64x2(8 * 100, 100)
    p.softmax_scale = 128 ** -0.5
    p.workspace = 0x40000
    p.workspace_bytes = fa.fa_bwd_workspace_size(2, 8, 100)
    return p


def test_bwd_validator(lib):
    assert fa.fa_check_bwd_params(good_bwd()) == fa.FA_OK
    assert fa.fa_bwd_workspace_size(2, 8, 100) >= 2 * 8 * 100 * 4
    assert fa.fa_bwd_workspace_size(1, 0, 10) == 0


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "dtype", fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "d", 64), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "Hkv", 3), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "dout", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "lse", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "lse", 0x20002), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "dk", 0x10008), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "workspace_bytes", 16), fa.FA_ERR_WORKSPACE),
    (lambda p: setattr(p, "workspace", 0x40004), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "softmax_scale", 0.0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "dq_strides", fa.I64x3(8 * 100 * 128, 100 * 128, 120)), fa.FA_ERR_INVALID_ARG),
])
def test_bwd_validator_errors(lib, mutate, status):
    p = good_bwd()
    mutate(p)
    assert fa.fa_check_bwd_params(p) == status


def test_bwd_wave_pingpong_validation(lib):
    p = good_bwd()
    p.wave_pingpong = 1
    assert fa.fa_check_bwd_params(p) == fa.FA_OK
    p.wave_pingpong = 2
    assert fa.fa_check_bwd_params(p) == fa.FA_ERR_INVALID_ARG
    assert "wave_pingpong" in fa.fa_last_error()


def good_quant():
    p = fa.FaFp8QuantParams()
    p.x, p.codes, p.scales, p.signs = 0x10000, 0x20000, 0x30000, 0
    p.in_dtype = fa.FA_BF16
    p.B, p.H, p.S, p.d = 2, 4, 130, 128
    p.x_strides = fa.I64x3(4 * 130 * 128, 130 * 128, 128)
    p.codes_strides = fa.I64x3(4 * 130 * 128, 130 * 128, 128)
    return p


def test_fp8_quant_validator(lib):
    assert fa.fa_check_fp8_quant_params(good_quant()) == fa.FA_OK


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "in_dtype", fa.FA_FP8_E4M3), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "d", 64), fa.FA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "x", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "scales", 0), fa.FA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "scales", 0x30002), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "signs", 0x40001), fa.FA_ERR_ALIGNMENT),
    (lambda p: setattr(p, "codes_strides", fa.I64x3(4 * 130 * 128, 130 * 128, 120)), fa.FA_ERR_ALIGNMENT),
])
def test_fp8_quant_validator_errors(lib, mutate, status):
    p = good_quant()
    mutate(p)
    assert fa.fa_check_fp8_quant_params(p) == status


def test_fwd_block_descales_validation(lib):
    p = good_fwd()
    p.in_dtype, p.out_dtype = fa.FA_FP8_E4M3, fa.FA_BF16
    for name in ("q_strides", "k_strides", "v_strides"):
        setattr(p, name, fa.I64x3(8 * 100 * 128, 100 * 128, 128))
    p.o_strides = fa.I64x3(8 * 100 * 128, 100 * 128, 128)
    p.q_block_descale = p.k_block_descale = p.v_block_descale = 0x50000
    p.q_descale = p.k_descale = p.v_descale = 0.0  # ignored with block descales
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p.v_block_descale = 0
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_INVALID_ARG
    p.v_block_descale = 0x50002
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_ALIGNMENT
    q = good_fwd()
    q.q_block_descale = q.k_block_descale = q.v_block_descale = 0x50000
    assert fa.fa_check_fwd_params(q) == fa.FA_ERR_INVALID_ARG  # bf16 inputs take no descales


def test_fwd_fp8_head_dim_and_p_precision(lib):
    # the host check predicts the launcher: fp8 has a kernel for d = 128 only
    p = good_fwd()
    p.in_dtype = fa.FA_FP8_E4M3
    p.q_descale = p.k_descale = p.v_descale = 1.0
    for n in ("q_strides", "k_strides", "v_strides"):
        setattr(p, n, fa.I64x3(8 * 100 * 128, 100 * 128, 128))
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    for pb in (0, 1):
        p.fp8_p_bf16 = pb
        assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p.fp8_p_bf16 = 2
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_INVALID_ARG
    p.fp8_p_bf16 = 0
    p.d = 64
    for n in ("q_strides", "k_strides", "v_strides", "o_strides"):
        setattr(p, n, fa.I64x3(8 * 100 * 64, 100 * 64, 64))
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_UNSUPPORTED
    assert "128" in fa.fa_last_error()
    q = good_fwd()
    q.fp8_p_bf16 = 1  # bf16 inputs: the flag has no meaning
    assert fa.fa_check_fwd_params(q) == fa.FA_ERR_INVALID_ARG


def test_fa_log_prints_the_launch(lib, tmp_path):
    """FA_LOG=1 prints the chosen kernel, grid, block and LDS bytes before the
    launch.  Run in a child process with no GPU visible, where the launch
    itself then fails with FA_ERR_HIP after the line is printed."""
    import subprocess
    import sys

    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("needs a process without a GPU: the call below passes fake device pointers")
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import tiled_exact_attention_fa_amd as fa\n"
        "sys.path.insert(0, " + repr(os.path.join(ROOT, "tests")) + ")\n"
        "from test_abi import good_fwd\n"
        "p = good_fwd(); p.causal = 1\n"
        "print('status', fa.load().fa_fwd(ctypes.byref(p), None))\n"
    )
    env = dict(os.environ, FA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert f"status {fa.FA_ERR_HIP}" in r.stdout
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[fa] ")]
    assert len(lines) == 1, r.stderr
    ln = lines[0]
    # 2 batches x 8 heads x one 256-row block of 100 rows
    assert ln.startswith("[fa] fwd_mfma16_kernel grid=16 block=512 lds=")
    assert "dtype=bf16 d=128 causal=1 B=2 Hq=8 G=4 Sq=100 Sk=100" in ln
    r0 = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, FA_LOG="0"), capture_output=True,
                        text=True, timeout=120)
    assert "[fa] " not in r0.stderr


# ---- the binding's own checks (the C ABI cannot see tensor shapes) -----------

def _cpu(shape, dtype=None):
    import torch

    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _fwd_set():
    import torch

    q, k, v = _cpu((2, 8, 100, 128)), _cpu((2, 2, 100, 128)), _cpu((2, 2, 100, 128))
    o, lse = _cpu((2, 8, 100, 128)), _cpu((2, 8, 100), torch.float32)
    return dict(q=q, k=k, v=v, o=o, lse=lse)


def test_binding_fwd_rejects_mismatches():
    import torch

    bad = [
        ("v", _cpu((2, 2, 99, 128)), ValueError),            # shorter V: read past its end
        ("o", _cpu((2, 8, 99, 128)), ValueError),            # shorter O: written past its end
        ("k", _cpu((2, 2, 100, 128), torch.float16), TypeError),
        ("o", _cpu((2, 8, 100, 128), torch.float16), TypeError),
        ("lse", _cpu((2, 8, 100)), TypeError),               # bf16 lse gets 4-byte writes
        ("lse", _cpu((2, 8, 100, 2), torch.float32)[..., 0], ValueError),  # sequence stride 2
        ("q", _cpu((2, 8, 100, 128), torch.int8), TypeError),
    ]
    for name, t, exc in bad:
        x = _fwd_set()
        x[name] = t
        with pytest.raises(exc):
            fa.fwd_params(**x)
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.fwd_params(**_fwd_set())


def test_binding_fwd_block_descales_checked():
    import torch

    x = _fwd_set()
    for n in ("q", "k", "v"):
        x[n] = x[n].to(torch.float8_e4m3fn)
    good = (_cpu((2, 8, 2), torch.float32), _cpu((2, 2, 2), torch.float32), _cpu((2, 2, 2), torch.float32))
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.fwd_params(**x, block_descales=good)
    with pytest.raises(ValueError):
        fa.fwd_params(**x, block_descales=(good[0], good[1], _cpu((2, 2, 1), torch.float32)))
    with pytest.raises(TypeError):
        fa.fwd_params(**x, block_descales=(good[0], good[1], _cpu((2, 2, 2))))


def _decode_set():
    import torch

    B, Hq, Hkv, L = 3, 8, 2, 64
    return dict(q=_cpu((B, Hq, 128)), k_cache=_cpu((B, Hkv, L, 128), torch.int8),
                v_cache=_cpu((B, Hkv, L, 128), torch.int8), k_scale=_cpu((B, Hkv, L), torch.float16),
                v_scale=_cpu((B, Hkv, L), torch.float16), o=_cpu((B, Hq, 128)),
                lse=_cpu((B, Hq), torch.float32), seq_lens=torch.full((B,), L, dtype=torch.int32))


def test_binding_decode_rejects_mismatches():
    import torch

    bad = [
        ("seq_lens", torch.full((3,), 64, dtype=torch.int64), TypeError),  # int64 would be misread
        ("seq_lens", torch.full((2,), 64, dtype=torch.int32), ValueError),
        ("v_cache", _cpu((3, 2, 63, 128), torch.int8), ValueError),
        ("v_cache", _cpu((3, 2, 64, 128), torch.uint8), TypeError),
        ("k_scale", _cpu((3, 2, 64), torch.float32), TypeError),
        ("o", _cpu((3, 8, 128), torch.float16), TypeError),
        ("lse", _cpu((3, 8)), TypeError),
        ("q", _cpu((3, 8, 128), torch.float16), TypeError),
    ]
    for name, t, exc in bad:
        x = _decode_set()
        x[name] = t
        with pytest.raises(exc):
            fa.decode_params(**x)
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.decode_params(**_decode_set())
    x = _decode_set()
    with pytest.raises(TypeError):   # window lengths must be int32 too
        fa.decode_params(**x, k_recent=_cpu((3, 2, 4, 128)), v_recent=_cpu((3, 2, 4, 128)),
                         recent_lens=torch.zeros(3, dtype=torch.int64))


def test_binding_bwd_append_quant_reject_mismatches():
    import torch

    q, k = _cpu((1, 4, 50, 128)), _cpu((1, 2, 50, 128))
    args = dict(q=q, k=k, v=k.clone(), o=q.clone(), dout=q.clone(), lse=_cpu((1, 4, 50), torch.float32),
                dq=q.clone(), dk=k.clone(), dv=k.clone())
    for name, t, exc in [("dv", _cpu((1, 2, 49, 128)), ValueError), ("lse", _cpu((1, 4, 50)), TypeError),
                         ("dout", _cpu((1, 4, 50, 128), torch.float16), TypeError)]:
        x = dict(args)
        x[name] = t
        with pytest.raises(exc):
            fa.bwd_params(**x)
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.bwd_params(**args)

    ap = dict(k_new=_cpu((2, 2, 5, 128)), v_new=_cpu((2, 2, 5, 128)), k_cache=_cpu((2, 2, 16, 128), torch.int8),
              v_cache=_cpu((2, 2, 16, 128), torch.int8), k_scale=_cpu((2, 2, 16), torch.float16),
              v_scale=_cpu((2, 2, 16), torch.float16), positions=torch.zeros(2, dtype=torch.int32))
    for name, t, exc in [("positions", torch.zeros(2, dtype=torch.int64), TypeError),
                         ("v_new", _cpu((2, 2, 4, 128)), ValueError),
                         ("v_scale", _cpu((2, 2, 15), torch.float16), ValueError)]:
        x = dict(ap)
        x[name] = t
        with pytest.raises(exc):
            fa.kv_append_params(**x)
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.kv_append_params(**ap)

    qp = dict(x=_cpu((1, 2, 70, 128)), codes=_cpu((1, 2, 70, 128), torch.uint8),
              scales=_cpu((1, 2, 2), torch.float32))
    for name, t, exc in [("scales", _cpu((1, 2, 1), torch.float32), ValueError),
                         ("codes", _cpu((1, 2, 70, 128), torch.int8), TypeError),
                         ("signs", _cpu((64,), torch.float32), ValueError)]:
        x = dict(qp)
        x[name] = t
        with pytest.raises(exc):
            fa.fp8_quant_params(**x)
    with pytest.raises(ValueError, match="not on a GPU"):
        fa.fp8_quant_params(**qp)


def test_decode_noalloc_refuses_before_any_hip_call(lib):
    # partials of 64 splits x 64 x 32 heads exceed the fixed scratch: the size
    # is checked on the host before the scratch is looked up or anything runs
    p = good_decode()
    p.B, p.Hq, p.Hkv, p.num_splits = 64, 32, 8, 64
    p.workspace, p.workspace_bytes = 0, 0
    assert fa.fa_decode_workspace_size(64, 32, 128, 64) > fa.FA_DECODE_NOALLOC_MAX_BYTES
    assert lib.fa_decode_kvq_noalloc(ctypes.byref(p), None) == fa.FA_ERR_WORKSPACE
    assert "scratch" in fa.fa_last_error()


def test_fwd_soft_exp2_validation(lib):
    p = good_fwd()
    p.soft_exp2 = 1
    assert fa.fa_check_fwd_params(p) == fa.FA_OK
    p.soft_exp2 = 3
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_INVALID_ARG
    p.soft_exp2 = 1
    p.d = 64
    for n in ("q_strides", "k_strides", "v_strides", "o_strides"):
        setattr(p, n, fa.I64x3(8 * 100 * 64, 100 * 64, 64))
    assert fa.fa_check_fwd_params(p) == fa.FA_ERR_UNSUPPORTED

