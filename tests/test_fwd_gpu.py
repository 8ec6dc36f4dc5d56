"""GPU parity of fa_fwd against the float64 oracle (through the C ABI).

Small shapes cover several tiles, ragged tails, Sq != Sk, grouped-query heads
and both head dims; every output buffer is pre-filled with NaN and surrounded
by guard bands, so unwritten or out-of-bounds elements are caught.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {  # max abs error bars: O, LSE
    "f32": (1e-4, 1e-4),
    "bf16": (2e-2, 1e-3),
    "f16": (2e-2, 1e-3),
}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
GUARD = 256


def guarded(shape, dtype, fill=float("nan")):
    """A tensor of `shape` inside a larger buffer whose guard bands hold a sentinel."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + n].view(shape)


def guards_intact(buf, fill_is_nan=True):
    g = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    return bool(torch.isnan(g).all()) if fill_is_nan else True


def run_fwd(fa, q, k, v, causal, out_dtype, scale=None, lse_wanted=True):
    B, Hq, Sq, d = q.shape
    obuf, o = guarded((B, Hq, Sq, d), out_dtype)
    lbuf, lse = guarded((B, Hq, Sq), torch.float32) if lse_wanted else (None, None)
    print(f"fa_fwd q={tuple(q.shape)} k={tuple(k.shape)} {q.dtype} causal={causal}", flush=True)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert guards_intact(obuf), "write outside O"
    if lbuf is not None:
        assert guards_intact(lbuf), "write outside LSE"
    return o, lse


def check(o, lse, q, k, v, causal, dt, scale=None):
    ro, rl = oracle.attention_fp64(q.cpu(), k.cpu(), v.cpu(), causal, scale)
    og = o.double().cpu().numpy()
    assert not np.isnan(og).any(), "unwritten O elements"
    tol_o, tol_l = TOL[dt]
    err_o = np.max(np.abs(og - ro)) if og.size else 0.0
    assert err_o <= tol_o, f"O max abs err {err_o}"
    if lse is not None:
        lg = lse.double().cpu().numpy()
        assert not np.isnan(lg).any(), "unwritten LSE elements"
        assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
        fin = np.isfinite(rl)
        err_l = np.max(np.abs(lg[fin] - rl[fin])) if fin.any() else 0.0
        assert err_l <= tol_l, f"LSE max abs err {err_l}"
    return err_o


def make(B, Hq, Hkv, Sq, Sk, d, dt, seed=0):
    cfg = fa_inputs.FwdConfig("t", dt, B, Hq, Hkv, Sq, Sk, d, False)
    x = fa_inputs.make_fwd_inputs(cfg, seed=seed)
    return [x[n].cuda() for n in ("q", "k", "v")]


SHAPES = [
    # B, Hq, Hkv, Sq, Sk
    (1, 1, 1, 1, 1),
    (1, 2, 2, 17, 17),
    (2, 2, 1, 64, 64),
    (1, 4, 1, 127, 127),
    (1, 1, 1, 128, 128),
    (1, 2, 2, 129, 129),
    (1, 8, 2, 300, 300),
    (2, 2, 2, 100, 260),   # Sq < Sk
    (1, 2, 2, 260, 100),   # Sq > Sk: causal leaves leading rows empty
    # 136 (batch, head) pairs: 17 per XCD, so the causal issue order of short
    # heads cuts each XCD's range into a group of 16 heads and a ragged group
    # of one; 17 is not a multiple of G = 4, so on most XCDs the groups
    # straddle K/V heads (a locality cost only: the mapping stays one-to-one)
    (2, 68, 17, 300, 300),
]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_small_shapes(gpu, dt, d, causal, shape):
    B, Hq, Hkv, Sq, Sk = shape
    q, k, v = make(B, Hq, Hkv, Sq, Sk, d, dt, seed=Sq * 7 + d)
    o, lse = run_fwd(gpu, q, k, v, causal, TDT[dt])
    check(o, lse, q, k, v, causal, dt)


def test_fwd_config_fp32_s128_d64(gpu):
    cfg = fa_inputs.CONFIGS["fp32_s128_d64"]
    x = fa_inputs.make_fwd_inputs(cfg, seed=0)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, lse = run_fwd(gpu, q, k, v, cfg.causal, torch.float32, cfg.scale)
    err = check(o, lse, q, k, v, cfg.causal, "f32", cfg.scale)
    print("fp32 config max abs err", err)


def test_fwd_no_lse_and_strided_layout(gpu):
    # BSHD storage viewed as BHSD: sequence stride H*d, head stride d
    B, H, S, d = 2, 4, 150, 128
    base = torch.randn(B, S, H, d, device="cuda").to(torch.bfloat16)
    q = base.transpose(1, 2)
    k = torch.randn(B, S, H, d, device="cuda").to(torch.bfloat16).transpose(1, 2)
    v = torch.randn(B, S, H, d, device="cuda").to(torch.bfloat16).transpose(1, 2)
    o = torch.full((B, S, H, d), float("nan"), device="cuda", dtype=torch.bfloat16).transpose(1, 2)
    gpu.fa_fwd(q, k, v, o, None, causal=True)
    torch.cuda.synchronize()
    check(o, None, q, k, v, True, "bf16")


NO_LSE_SHAPES = [(1, 2, 2, 64, 64), (2, 8, 2, 300, 300), (1, 4, 1, 130, 300), (1, 2, 2, 300, 130),
                 (1, 2, 2, 1, 1), (1, 4, 4, 1024, 1024)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", NO_LSE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_without_lse_output(gpu, dt, causal, shape):
    """With no LSE pointer the d = 128 kernel skips the unrounded row sum; O
    is divided by the rounded sum either way, so O must equal the O of the
    call with an LSE output bit for bit, and meet the oracle's bar."""
    B, Hq, Hkv, Sq, Sk = shape
    q, k, v = make(B, Hq, Hkv, Sq, Sk, 128, dt, seed=Sq + 3 * Sk)
    o_l, lse = run_fwd(gpu, q, k, v, causal, TDT[dt])
    o_n, none = run_fwd(gpu, q, k, v, causal, TDT[dt], lse_wanted=False)
    assert none is None
    assert torch.equal(o_n, o_l), "O differs between the calls with and without an LSE output"
    check(o_n, None, q, k, v, causal, dt)


MORE_CASES = [
    # name, B, Hq, Hkv, Sq, Sk, factor on Q and K, softmax scale (None: 1/sqrt(d))
    ("group8", 1, 16, 2, 300, 300, 1.0, None),
    ("group16", 2, 32, 2, 200, 200, 1.0, None),
    ("mqa32", 1, 32, 1, 260, 260, 1.0, None),
    ("short_q_long_k", 1, 4, 2, 64, 4100, 1.0, None),     # 65 key tiles, one partial
    ("long_q_short_k", 1, 2, 1, 1100, 70, 1.0, None),     # causal: 1030 rows see no key
    ("peaked", 1, 4, 2, 300, 300, 4.0, None),             # scores span about +-64: one-hot rows, lazy max moves
    ("flat", 1, 4, 2, 300, 300, 1.0, 0.01),               # nearly uniform rows
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", MORE_CASES, ids=lambda c: c[0])
def test_fwd_groups_lengths_and_score_ranges(gpu, dt, causal, case):
    """Wider query groups (8, 16, 32 query heads per K/V head), a short query
    block against many key tiles and the reverse, and score distributions at
    both ends: strongly peaked rows (the running max moves by large steps, and
    O is close to a single V row) and nearly uniform ones."""
    name, B, Hq, Hkv, Sq, Sk, f, scale = case
    q, k, v = make(B, Hq, Hkv, Sq, Sk, 128, dt, seed=Sq + Sk + Hq)
    if f != 1.0:
        q = (q.float() * f).to(q.dtype)
        k = (k.float() * f).to(k.dtype)
    o, lse = run_fwd(gpu, q, k, v, causal, TDT[dt], scale)
    check(o, lse, q, k, v, causal, dt, scale)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(1024, 1024), (1025, 1025), (700, 1024), (1024, 1025)])
def test_fwd_d64_launch_choice(gpu, dt, causal, Sq, Sk):
    """d = 64 runs 128-row workgroups (two per compute unit) up to 1024 keys and
    256-row ones past that: both sides of the switch, and Sq != Sk across it."""
    q, k, v = make(2, 4, 2, Sq, Sk, 64, dt, seed=Sq + 2 * Sk)
    o, lse = run_fwd(gpu, q, k, v, causal, TDT[dt])
    check(o, lse, q, k, v, causal, dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(512, 512), (513, 513), (300, 512), (512, 513)])
def test_fwd_d128_launch_choice(gpu, dt, causal, Sq, Sk):
    """d = 128 with an LSE output runs 128-row workgroups up to 512 keys and
    256-row ones past that (and without an LSE output, 256-row ones
    throughout): both sides of the switch, Sq != Sk across it, and the no-LSE
    call at the same sizes."""
    q, k, v = make(2, 4, 2, Sq, Sk, 128, dt, seed=Sq + 3 * Sk)
    o, lse = run_fwd(gpu, q, k, v, causal, TDT[dt])
    check(o, lse, q, k, v, causal, dt)
    o2, _ = run_fwd(gpu, q, k, v, causal, TDT[dt], lse_wanted=False)
    check(o2, None, q, k, v, causal, dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 17, 600), (2, 4, 1, 129, 700), (1, 4, 2, 300, 577), (1, 2, 1, 700, 600)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fwd_d128_ragged_past_512_keys(gpu, dt, causal, shape):
    """Ragged query and key lengths just past 512 keys, so the 256-row
    workgroups see partial last tiles, short query blocks and (causal, Sq > Sk)
    leading rows that see no key."""
    B, Hq, Hkv, Sq, Sk = shape
    q, k, v = make(B, Hq, Hkv, Sq, Sk, 128, dt, seed=Sq * 7 + Sk)
    o, lse = run_fwd(gpu, q, k, v, causal, TDT[dt])
    check(o, lse, q, k, v, causal, dt)


def test_fwd_deterministic(gpu):
    q, k, v = make(2, 8, 2, 333, 333, 128, "bf16", seed=11)
    o1, l1 = run_fwd(gpu, q, k, v, True, torch.bfloat16)
    o2, l2 = run_fwd(gpu, q, k, v, True, torch.bfloat16)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_fwd_gqa_equals_repeated_heads(gpu):
    q, k, v = make(1, 8, 2, 200, 200, 128, "bf16", seed=12)
    o1, l1 = run_fwd(gpu, q, k, v, True, torch.bfloat16)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = run_fwd(gpu, q, kr, vr, True, torch.bfloat16)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_fwd_constant_v_and_zero_q(gpu):
    B, H, S, d = 1, 2, 190, 64
    q = torch.zeros(B, H, S, d, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(B, H, S, d, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, H, 1, d, device="cuda").to(torch.bfloat16).expand(B, H, S, d).contiguous()
    o, lse = run_fwd(gpu, q, k, v, True, torch.bfloat16)
    assert torch.equal(o, v), "constant V must come back exactly"
    want = torch.log(torch.arange(1, S + 1, device="cuda", dtype=torch.float32))
    assert float((lse[0, 0] - want).abs().max()) < 1e-5


def test_fwd_rejects_bad_params(gpu):
    q, k, v = make(1, 4, 3, 16, 16, 128, "bf16")[0], None, None
    k = torch.zeros(1, 3, 16, 128, device="cuda", dtype=torch.bfloat16)
    o = torch.empty_like(q)
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_fwd(q, k, k, o)  # 4 query heads over 3 kv heads
    assert e.value.status == gpu.FA_ERR_INVALID_ARG
    q96 = torch.zeros(1, 1, 8, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_fwd(q96, q96, q96, torch.empty_like(q96))
    assert e.value.status == gpu.FA_ERR_UNSUPPORTED


# ---- fp8 e4m3 inputs (per-tensor descales), bf16 output ----------------------

FP8_TOL_O = 8e-2   # fp8 path bar; the oracle sees the same e4m3 codes x descales
FP8_SHAPES = [
    (1, 1, 1, 1, 1),
    (1, 2, 2, 64, 64),
    (2, 2, 1, 129, 129),
    (1, 4, 2, 300, 300),
    (1, 2, 2, 100, 260),
    (1, 2, 2, 260, 100),
    (2, 68, 17, 300, 300),  # grouped causal order with a ragged last group
]


def fp8_oracle_inputs(x):
    from oracle.e4m3 import e4m3_decode

    return (e4m3_decode(x["q"].cpu()) * x["q_scale"], e4m3_decode(x["k"].cpu()) * x["k_scale"],
            e4m3_decode(x["v"].cpu()) * x["v_scale"])


def run_fp8(fa, x, causal, p_bf16=False):
    q, k, v = x["q"], x["k"], x["v"]
    B, Hq, Sq, d = q.shape
    obuf, o = guarded((B, Hq, Sq, d), torch.bfloat16)
    lbuf, lse = guarded((B, Hq, Sq), torch.float32)
    print(f"fa_fwd fp8 q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} p_bf16={p_bf16}", flush=True)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, q_descale=x["q_scale"], k_descale=x["k_scale"],
              v_descale=x["v_scale"], p_bf16=p_bf16)
    torch.cuda.synchronize()
    assert guards_intact(obuf) and guards_intact(lbuf)
    return o, lse


@pytest.mark.parametrize("p_bf16", [False, True], ids=["p_e4m3", "p_bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_fp8_small(gpu, causal, shape, p_bf16):
    B, Hq, Hkv, Sq, Sk = shape
    cfg = fa_inputs.FwdConfig("t", "fp8", B, Hq, Hkv, Sq, Sk, 128, causal)
    x = {n: (t.cuda() if torch.is_tensor(t) else t) for n, t in fa_inputs.make_fwd_inputs(cfg, seed=Sq).items()}
    o, lse = run_fp8(gpu, x, causal, p_bf16)
    qf, kf, vf = fp8_oracle_inputs(x)
    ro, rl = oracle.attention_fp64(qf, kf, vf, causal)
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert not np.isnan(og).any() and not np.isnan(lg).any()
    err = float(np.max(np.abs(og - ro)))
    assert err <= FP8_TOL_O, f"O err {err}"
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert float(np.max(np.abs(lg[fin] - rl[fin]), initial=0.0)) <= 1e-3
    print("fp8 max |dO|", err)


# ---- full-size workloads, every output element checked --------------------

FULL = [("bf16_b4_h16_s2048_causal", False), ("bf16_gqa32x8_s16384_causal_outlier", False),
        ("fp8_b8_h16_s4096", False), ("fp8_b8_h16_s4096", True)]


@pytest.mark.parametrize("name,p_bf16", FULL, ids=["bf16_s2048", "bf16_gqa_s16384", "fp8_p_e4m3", "fp8_p_bf16"])
def test_fwd_full_size(gpu, name, p_bf16):
    """The three prefill workloads at full size, in the launch configuration
    the benchmark times, compared with the float64 oracle element by element:
    every O and every LSE value.  The long-context workload is the only one
    whose heads have more than 8 query blocks (one longest-first issue order
    over 256 key tiles), so this is its only parity case."""
    cfg = fa_inputs.CONFIGS[name]
    x = fa_inputs.make_fwd_inputs(cfg, seed=0, device="cuda")
    odt = torch.float32 if cfg.dtype == "f32" else (torch.float16 if cfg.dtype == "f16" else torch.bfloat16)
    o = torch.full((cfg.B, cfg.Hq, cfg.Sq, cfg.d), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((cfg.B, cfg.Hq, cfg.Sq), float("nan"), device="cuda")
    print(f"fa_fwd full-size {name}", flush=True)
    gpu.fa_fwd(x["q"], x["k"], x["v"], o, lse, causal=cfg.causal, softmax_scale=cfg.scale,
               q_descale=x.get("q_scale", 1.0), k_descale=x.get("k_scale", 1.0),
               v_descale=x.get("v_scale", 1.0), p_bf16=p_bf16)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()) and not bool(torch.isnan(lse).any())
    if cfg.dtype == "fp8":
        qf, kf, vf = fp8_oracle_inputs(x)
    else:
        qf, kf, vf = (x[n].cpu() for n in ("q", "k", "v"))
    del x
    if cfg.dtype in ("bf16", "f16"):
        # the same call without an LSE output (the kernel then skips the
        # unrounded row sum) must give the same O, bit for bit
        o_n = torch.full_like(o, float("nan"))
        gpu.fa_fwd(qf.cuda(), kf.cuda(), vf.cuda(), o_n, None, causal=cfg.causal, softmax_scale=cfg.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o), f"{name}: O differs between the calls with and without an LSE output"
        del o_n
    ro, rl = oracle.attention_fp64(qf, kf, vf, cfg.causal, cfg.scale)
    og = o.double().cpu().numpy()
    lg = lse.double().cpu().numpy()
    err_o = float(np.max(np.abs(og - ro)))
    err_l = float(np.max(np.abs(lg - rl)))
    print(f"{name} p_bf16={p_bf16}: every element, max|dO|={err_o:.3g} max|dLSE|={err_l:.3g}", flush=True)
    assert err_o <= (FP8_TOL_O if cfg.dtype == "fp8" else 2e-2) and err_l <= 1e-3


# ---- software exponentials (a quarter of them on the FMA pipe) --------------

SOFT_SHAPES = [(1, 2, 2, 64, 64), (1, 8, 2, 300, 300), (2, 2, 2, 100, 260), (1, 2, 2, 260, 100)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SOFT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_soft_exp2(gpu, dt, causal, shape):
    """soft_exp2 = 1: same bars as the hardware exponentials, including rows
    that see no key (Sq > Sk, causal), whose probabilities must stay 0."""
    B, Hq, Hkv, Sq, Sk = shape
    q, k, v = make(B, Hq, Hkv, Sq, Sk, 128, dt, seed=Sq + 5)
    obuf, o = guarded((B, Hq, Sq, 128), TDT[dt])
    lbuf, lse = guarded((B, Hq, Sq), torch.float32)
    print(f"fa_fwd soft_exp2 q={tuple(q.shape)} k={tuple(k.shape)} {dt} causal={causal}", flush=True)
    gpu.fa_fwd(q, k, v, o, lse, causal=causal, soft_exp2=True)
    torch.cuda.synchronize()
    assert guards_intact(obuf) and guards_intact(lbuf)
    check(o, lse, q, k, v, causal, dt)


def test_fwd_soft_exp2_full_size(gpu):
    """The long-context workload with soft_exp2 = 1, every element."""
    cfg = fa_inputs.CONFIGS["bf16_gqa32x8_s16384_causal_outlier"]
    x = fa_inputs.make_fwd_inputs(cfg, seed=0, device="cuda")
    o = torch.full((cfg.B, cfg.Hq, cfg.Sq, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((cfg.B, cfg.Hq, cfg.Sq), float("nan"), device="cuda")
    print("fa_fwd full-size soft_exp2", flush=True)
    gpu.fa_fwd(x["q"], x["k"], x["v"], o, lse, causal=True, soft_exp2=True)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()) and not bool(torch.isnan(lse).any())
    ro, rl = oracle.attention_fp64(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True)
    err_o = float(np.max(np.abs(o.double().cpu().numpy() - ro)))
    err_l = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    print(f"soft_exp2 long-context, every element: max|dO|={err_o:.3g} max|dLSE|={err_l:.3g}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3

