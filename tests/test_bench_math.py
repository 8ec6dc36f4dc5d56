"""Algorithmic-work formulas used by bench.py, against hand-computed values."""

import dataclasses

import bench
import fa_inputs

C = fa_inputs.CONFIGS


def test_visible_pairs():
    assert bench.visible_pairs(4, 4, False) == 16
    assert bench.visible_pairs(4, 4, True) == 10          # 1+2+3+4
    assert bench.visible_pairs(2, 5, True) == 4 + 5       # bottom-right: rows see 4 and 5 keys
    assert bench.visible_pairs(5, 2, True) == 0 + 0 + 0 + 1 + 2


def test_prefill_flops():
    assert bench.fwd_flops(C["bf16_b4_h16_s2048_causal"]) == 4 * 128 * 4 * 16 * 2048 * 2049 // 2
    assert bench.fwd_flops(C["bf16_gqa32x8_s16384_causal_outlier"]) == 2199157473280
    assert bench.fwd_flops(C["fp8_b8_h16_s4096"]) == 4 * 8 * 16 * 128 * 4096 * 4096
    assert bench.fwd_flops(C["fp32_s128_d64"]) == 4 * 64 * 128 * 128


def test_decode_bytes():
    c = C["decode_int8_b64_gqa32x8_L32768"]
    kv = 2 * 1 * 64 * 32768 * 8 * 128 * 1          # 2 * layers * batch * tokens * kv_heads * d * 1 byte
    assert kv == 4294967296
    assert bench.decode_bytes(c) == kv + 67108864 + 524288 + 524288 + 8192 == 4363132928
    small = dataclasses.replace(c, B=1, Hq=4, Hkv=1, L=10)
    assert bench.decode_bytes(small) == 2 * 10 * 128 + 2 * 10 * 2 + 4 * 128 * 2 * 2 + 4 * 4


def test_gpus_above_one_is_refused():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
