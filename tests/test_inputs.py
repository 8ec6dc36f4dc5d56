"""The seeded input generators and input-side quantisers (CPU only)."""

import dataclasses

import numpy as np
import torch

import fa_inputs
from oracle.e4m3 import e4m3_decode


def test_int8_tokhead_quantiser_bounds():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(2, 3, 50, 128, generator=g)
    x[0, 0, 7] = 0.0  # an all-zero token gets scale 0 and codes 0
    codes, sc = fa_inputs.quantize_int8_tokhead(x)
    assert codes.dtype == torch.int8 and sc.dtype == torch.float16
    assert int(codes.abs().max()) <= 127
    assert float(sc[0, 0, 7]) == 0.0 and int(codes[0, 0, 7].abs().max()) == 0
    assert torch.equal(sc, (x.abs().amax(-1) / 127).to(torch.float16))
    err = (x.double() - codes.double() * sc.double()[..., None]).abs()
    assert bool((err <= sc.double()[..., None] / 2 * (1 + 1e-6) + 1e-12).all())


def test_fp8_quantiser_scale_absmax_and_rounding():
    g = torch.Generator().manual_seed(4)
    x = torch.randn(4, 1000, generator=g)
    codes, s = fa_inputs.quantize_fp8_per_tensor(x)
    assert s == float((x.abs().max() / 448.0).to(torch.float32))
    vals = e4m3_decode(codes)
    i = int(x.abs().argmax())
    assert abs(vals.reshape(-1)[i]) == 448.0
    # round-to-nearest against the decoded table, brute force over all codes
    table = e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(table)
    y = (x.double() / s).numpy().reshape(-1)[:2000]
    got = vals.reshape(-1)[:2000]
    dist = np.abs(y[:, None] - table[None, finite])
    best = dist.min(axis=1)
    assert np.all(np.abs(np.abs(y - got) - best) <= 1e-12 * np.maximum(1, np.abs(y)))


def test_outlier_rows_exactly_one_percent_times_eight():
    cfg = dataclasses.replace(fa_inputs.CONFIGS["bf16_gqa32x8_s16384_causal_outlier"],
                              Hq=4, Hkv=2, Sq=300, Sk=300, d=16)
    a = fa_inputs.make_fwd_inputs(cfg, seed=0)
    plain = dataclasses.replace(cfg, outlier_frac=0.0)
    b = fa_inputs.make_fwd_inputs(plain, seed=0)
    assert torch.equal(a["q"], b["q"])
    ratio = a["k"].float() / b["k"].float()
    rows = (ratio.abs() > 4).all(dim=-1)  # outlier rows are x8 in every channel
    assert rows.sum(dim=-1).tolist() == [[3, 3]]  # round(0.01 * 300) per kv head
    assert torch.allclose(ratio[rows], torch.full_like(ratio[rows], 8.0), rtol=0.02)
    assert torch.equal(a["k"][~rows], b["k"][~rows])


def test_generators_are_deterministic():
    cfg = dataclasses.replace(fa_inputs.CONFIGS["fp8_b8_h16_s4096"], B=1, Hq=2, Hkv=2, Sq=64, Sk=64)
    a = fa_inputs.make_fwd_inputs(cfg, seed=5)
    b = fa_inputs.make_fwd_inputs(cfg, seed=5)
    assert torch.equal(a["q"].view(torch.uint8), b["q"].view(torch.uint8)) and a["v_scale"] == b["v_scale"]
    dc = dataclasses.replace(fa_inputs.CONFIGS["decode_int8_b64_gqa32x8_L32768"], B=2, L=64)
    x = fa_inputs.make_decode_inputs(dc, seed=1)
    y = fa_inputs.make_decode_inputs(dc, seed=1)
    assert all(torch.equal(x[n], y[n]) for n in x)
    assert x["q"].shape == (2, 32, 128) and x["k"].shape == (2, 8, 64, 128)
    assert x["seq_lens"].tolist() == [64, 64]


def test_config_table_matches_workloads():
    c = fa_inputs.CONFIGS
    assert (c["fp32_s128_d64"].Sq, c["fp32_s128_d64"].d, c["fp32_s128_d64"].causal) == (128, 64, False)
    x = c["bf16_b4_h16_s2048_causal"]
    assert (x.B, x.Hq, x.Sq, x.d, x.causal) == (4, 16, 2048, 128, True)
    x = c["bf16_gqa32x8_s16384_causal_outlier"]
    assert (x.Hq, x.Hkv, x.Sq, x.outlier_frac) == (32, 8, 16384, 0.01)
    x = c["fp8_b8_h16_s4096"]
    assert (x.B, x.Hq, x.Sq, x.causal, x.dtype) == (8, 16, 4096, False, "fp8")
    x = c["decode_int8_b64_gqa32x8_L32768"]
    assert (x.B, x.Hq, x.Hkv, x.L, x.num_splits) == (64, 32, 8, 32768, 16)


def test_kv_generators_fp8_window_and_append():
    dc = fa_inputs.DecodeConfig("t", 2, 8, 2, 40, 128, 4, (40, 7), "fp8", 16, (16, 3))
    x = fa_inputs.make_decode_inputs(dc, seed=2)
    assert x["k"].dtype == torch.uint8 and x["k"].shape == (2, 2, 40, 128)
    assert x["k_recent"].dtype == torch.bfloat16 and x["k_recent"].shape == (2, 2, 16, 128)
    assert x["recent_lens"].tolist() == [16, 3] and x["seq_lens"].tolist() == [40, 7]
    # no NaN codes; each row's absmax maps to +-448
    assert not ((x["k"] & 0x7F) == 0x7F).any()
    assert bool((((x["v"] & 0x7F) == 0x7E).sum(dim=-1) >= 1).all())
    ac = fa_inputs.AppendConfig("a", 2, 3, 5, 16, 128, "int8", 4)
    y = fa_inputs.make_append_inputs(ac, seed=0)
    assert y["k_new"].shape == (2, 3, 5, 128) and y["k_cache"].dtype == torch.int8
    assert y["positions"].tolist() == [4, 4] and int(y["k_cache"].abs().max()) == 0


def test_kv_config_table():
    k = fa_inputs.KV_CONFIGS
    x = k["decode_fp8_b64_gqa32x8_L32768"]
    assert (x.B, x.Hq, x.Hkv, x.L, x.num_splits, x.kv_format, x.W) == (64, 32, 8, 32768, 16, "fp8", 0)
    x = k["decode_int8_window128_b64_gqa32x8_L32768"]
    assert (x.kv_format, x.W) == ("int8", 128)
    for f in ("int8", "fp8"):
        x = k[f"append_{f}_b64_h8_t4096"]
        assert (x.B, x.H, x.T, x.L, x.pos0, x.kv_format) == (64, 8, 4096, 32768, 28672, f)


def test_rotation_signs_and_quant_inputs():
    s = fa_inputs.make_rotation_signs(128, seed=3)
    assert s.dtype == torch.float32 and set(s.tolist()) == {-1.0, 1.0}
    assert torch.equal(s, fa_inputs.make_rotation_signs(128, seed=3))
    assert not torch.equal(s, fa_inputs.make_rotation_signs(128, seed=4))
    cfg = fa_inputs.QuantConfig("t", 1, 2, 70, 128, True)
    x = fa_inputs.make_quant_inputs(cfg, seed=1)
    assert x["q"].shape == (1, 2, 70, 128) and x["q"].dtype == torch.bfloat16
    assert torch.equal(x["signs"], fa_inputs.make_rotation_signs(128, seed=1))
    # the same bf16 draws as the forward recipe of that shape
    fx = fa_inputs.make_fwd_inputs(fa_inputs.FwdConfig("t", "bf16", 1, 2, 2, 70, 70, 128, False), seed=1)
    assert torch.equal(x["v"], fx["v"])
