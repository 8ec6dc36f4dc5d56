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


def test_kv_workload_bytes():
    k = fa_inputs.KV_CONFIGS
    base = bench.decode_bytes(C["decode_int8_b64_gqa32x8_L32768"])
    assert bench.decode_bytes(k["decode_fp8_b64_gqa32x8_L32768"]) == base  # 1-byte codes either way
    # the window adds its bf16 keys and values: 2 * B * Hkv * W * d * 2 bytes
    assert bench.decode_bytes(k["decode_int8_window128_b64_gqa32x8_L32768"]) == base + 2 * 64 * 8 * 128 * 128 * 2
    a = k["append_int8_b64_h8_t4096"]
    rows = 64 * 8 * 4096
    # bf16 rows read (K and V), one code byte per element and a 2-byte scale per row written
    assert bench.append_bytes(a) == 2 * rows * 256 + 2 * (rows * 128 + rows * 2) == 1619001344


def test_fp8_variant_workloads():
    v = fa_inputs.FP8_VARIANT_CONFIGS
    fb = v["fp8_block_rot_b8_h16_s4096"]
    # the block-scaled forward does the same work as the per-tensor one
    assert bench.fwd_flops(fb) == bench.fwd_flops(C["fp8_b8_h16_s4096"])
    assert bench.kernel_family(fb) == "fwd8"
    qc = v["fp8_quant_rot_b8_h16_s4096"]
    n = 8 * 16 * 4096 * 128
    # per tensor: 2-byte rows read, 1-byte codes and a 4-byte scale per 64 rows written
    assert bench.quant_bytes(qc) == 3 * (3 * n + 8 * 16 * 64 * 4)
    assert bench.kernel_family(qc) == "quant" and bench.workload(qc.name) is qc


def test_counter_digest_follows_each_kernel_family():
    fams = {n: bench.kernel_family(bench.workload(n)) for n in list(C) + list(fa_inputs.KV_CONFIGS)}
    assert fams["bf16_b4_h16_s2048_causal"] == "fwd16" and fams["fp8_b8_h16_s4096"] == "fwd8"
    assert fams["decode_fp8_b64_gqa32x8_L32768"] == "decode" and fams["append_fp8_b64_h8_t4096"] == "append"
    digests = {f: bench.source_digest(f) for f in bench.KERNEL_SOURCES}
    assert len(set(digests.values())) == len(digests)


def test_variant_workloads_are_benchmarked_with_their_switch():
    # the two-role backward runs the same work as the default backward
    pp = fa_inputs.BWD_VARIANT_CONFIGS["bwd_pingpong_bf16_gqa32x8_s16384_causal_outlier"]
    base = fa_inputs.BWD_CONFIGS["bwd_bf16_gqa32x8_s16384_causal_outlier"]
    assert isinstance(pp, fa_inputs.PingPongBwdConfig) and bench.workload(pp.name) is pp
    assert bench.bwd_flops(pp) == bench.bwd_flops(base) and bench.kernel_family(pp) == "bwd"


def test_host_description_fields():
    # the oracle baseline names the CPU it ran on (None only where /proc/cpuinfo has no model line)
    m = bench._cpu_model()
    assert m is None or (isinstance(m, str) and m)
    # without a readable GPU the amd-smi sample is empty, never an exception
    p, c = bench._smi_sample()
    assert (p is None or p > 0) and (c is None or c > 0)


def test_no_amd_smi_under_a_profiler(monkeypatch):
    # a profiled program must not start amd-smi (its child would carry the profiler's preload)
    monkeypatch.setenv("ROCPROFILER_LIBRARY_CTOR", "1")
    assert bench._under_profiler()
    assert bench._smi_sample() == (None, None)
    obs = bench.observed_clock(lambda: None, 1.0)
    assert obs["gfx_clock_mhz"] is None and obs["samples"] == 0
