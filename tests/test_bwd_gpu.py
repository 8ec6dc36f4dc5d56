"""GPU parity of fa_bwd (dQ, dK, dV by recomputation) against the float64
oracle's gradients, computed from the same bf16/fp16 inputs.

Tolerance: every gradient tensor must satisfy max |GPU - oracle| <= 2e-2 *
max |oracle| + 1e-4 over that tensor.  The kernels round P and dS to the input type
(relative 2^-9 for bf16) as matrix-core operands and the outputs to the input
type (another 2^-9 of the largest element); both are far inside the bar, while
any structural mistake (a wrong mask, a missing row term, a transposed operand)
moves results by a sizeable fraction of their scale."""

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2


def _dout(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)


def run_bwd(fa, x, dout, causal, scale=None):
    q, k, v = x["q"], x["k"], x["v"]
    B, Hq, Sq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
    print(f"fa_fwd+fa_bwd q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} {q.dtype}", flush=True)
    fa.fa_fwd(q, k, v, o, lse, causal=causal, softmax_scale=scale)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(got, ref, name):
    g = got.double().cpu().numpy()
    assert not np.isnan(g).any(), f"{name} has NaN"
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(g - ref)))
    # (the absolute floor only matters where the exact gradient is 0, as with
    # a single key: there the GPU result is rounding noise of the products)
    assert err <= REL_TOL * scale + 1e-4, f"{name}: max err {err:.3g} vs max |ref| {scale:.3g}"
    return err / max(scale, 1e-12)


CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, causal
    ("bf16", 1, 1, 1, 1, 1, False),
    ("bf16", 1, 2, 2, 64, 64, True),
    ("bf16", 2, 4, 2, 200, 200, True),     # GQA, ragged tiles
    ("bf16", 1, 4, 1, 130, 300, True),     # Sq < Sk (bottom-right diagonal)
    ("bf16", 1, 2, 2, 300, 130, True),     # Sq > Sk: leading rows see no key
    ("bf16", 2, 2, 1, 257, 129, False),
    ("fp16", 2, 4, 4, 192, 192, True),
    ("fp16", 1, 8, 2, 100, 333, False),
    ("bf16", 1, 2, 2, 1024, 1024, True),   # several 128-row / 128-key blocks
    ("bf16", 1, 16, 2, 200, 200, True),    # 8 query heads per K/V head
    ("fp16", 1, 16, 1, 150, 290, False),   # 16 query heads sharing one K/V head
]


@pytest.mark.parametrize("dt,B,Hq,Hkv,Sq,Sk,causal", CASES)
def test_bwd_small(gpu, dt, B, Hq, Hkv, Sq, Sk, causal):
    cfg = fa_inputs.FwdConfig("t", dt if dt == "bf16" else "f16", B, Hq, Hkv, Sq, Sk, 128, causal)
    xc = fa_inputs.make_fwd_inputs(cfg, seed=Sq + Sk)
    dout = _dout((B, Hq, Sq, 128), Sq * 7 + Sk, xc["q"].dtype)
    x = {n: xc[n].cuda() for n in ("q", "k", "v")}
    dq, dk, dv = run_bwd(gpu, x, dout.cuda(), causal)
    rq, rk, rv = oracle.attention_bwd_fp64(xc["q"], xc["k"], xc["v"], dout, causal)
    rel = [check(dq, rq, "dQ"), check(dk, rk, "dK"), check(dv, rv, "dV")]
    print("relative max errors dQ dK dV:", [f"{r:.2e}" for r in rel])


def test_bwd_deterministic_and_gqa_sums(gpu):
    # no atomics: two runs agree bit for bit; dK/dV of a shared kv head equal
    # the sum over its query heads of an MHA run with the kv head repeated
    cfg = fa_inputs.FwdConfig("t", "bf16", 1, 4, 2, 150, 150, 128, True)
    xc = fa_inputs.make_fwd_inputs(cfg, seed=3)
    dout = _dout((1, 4, 150, 128), 4, torch.bfloat16).cuda()
    x = {n: xc[n].cuda() for n in ("q", "k", "v")}
    a = run_bwd(gpu, x, dout, True)
    b = run_bwd(gpu, x, dout, True)
    for u, w in zip(a, b):
        assert torch.equal(u.view(torch.int16), w.view(torch.int16))
    xr = {"q": x["q"], "k": x["k"].repeat_interleave(2, dim=1).contiguous(),
          "v": x["v"].repeat_interleave(2, dim=1).contiguous()}
    c = run_bwd(gpu, xr, dout, True)
    assert torch.equal(a[0].view(torch.int16), c[0].view(torch.int16))  # dQ does not see the grouping
    for grouped, mha in ((a[1], c[1]), (a[2], c[2])):
        summed = mha.float().view(1, 2, 2, 150, 128).sum(dim=2)
        assert float((grouped.float() - summed).abs().max()) <= 2e-2 * float(summed.abs().max())


PINGPONG_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, causal
    ("bf16", 1, 2, 2, 64, 64, True),
    ("bf16", 2, 4, 2, 200, 200, True),
    ("bf16", 1, 4, 1, 130, 300, True),
    ("bf16", 1, 2, 2, 300, 130, True),
    ("bf16", 2, 2, 1, 257, 129, False),
    ("fp16", 1, 8, 2, 100, 333, False),
    ("bf16", 1, 4, 2, 1024, 1024, True),
    ("bf16", 1, 2, 1, 1000, 1100, False),
]


@pytest.mark.parametrize("dt,B,Hq,Hkv,Sq,Sk,causal", PINGPONG_CASES)
def test_bwd_wave_pingpong_bitwise(gpu, dt, B, Hq, Hkv, Sq, Sk, causal):
    # the two-role dK/dV schedule runs the same tiles in the same order in each
    # wave, so all three gradients equal the default schedule's bit for bit
    cfg = fa_inputs.FwdConfig("t", dt if dt == "bf16" else "f16", B, Hq, Hkv, Sq, Sk, 128, causal)
    xc = fa_inputs.make_fwd_inputs(cfg, seed=Sq + 3 * Sk)
    dout = _dout((B, Hq, Sq, 128), Sq + Sk, xc["q"].dtype).cuda()
    x = {n: xc[n].cuda() for n in ("q", "k", "v")}
    ref = run_bwd(gpu, x, dout, causal)
    o = torch.empty_like(x["q"])
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device="cuda")
    gpu.fa_fwd(x["q"], x["k"], x["v"], o, lse, causal=causal)
    got = [torch.full_like(t, float("nan")) for t in ref]
    print(f"fa_bwd wave_pingpong q={(B, Hq, Sq)} k={(Hkv, Sk)} causal={causal} {dt}", flush=True)
    gpu.fa_bwd(x["q"], x["k"], x["v"], o, dout, lse, *got, causal=causal, wave_pingpong=True)
    torch.cuda.synchronize()
    for name, u, w in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(u.view(torch.int16), w.view(torch.int16)), name
    if Sq * Sk <= 300 * 300:
        rq, rk, rv = oracle.attention_bwd_fp64(xc["q"], xc["k"], xc["v"], dout.cpu(), causal)
        check(got[0], rq, "dQ")
        check(got[1], rk, "dK")
        check(got[2], rv, "dV")


def test_bwd_strided_bshd(gpu):
    # token-major [B, S, H, d] buffers viewed as BHSD, for inputs and gradients
    B, S, H = 1, 96, 2
    g = torch.Generator().manual_seed(8)
    mk = lambda: torch.randn(B, S, H, 128, generator=g).to(torch.bfloat16).cuda()
    q, k, v, dout = mk(), mk(), mk(), mk()
    qv, kv, vv, dov = (t.permute(0, 2, 1, 3) for t in (q, k, v, dout))
    o = torch.empty_like(q).permute(0, 2, 1, 3)
    lse = torch.empty(B, H, S, device="cuda")
    print("fa_bwd BSHD strides", flush=True)
    gpu.fa_fwd(qv, kv, vv, o, lse, causal=True)
    dq = torch.empty_like(q).permute(0, 2, 1, 3)
    dk = torch.empty_like(k).permute(0, 2, 1, 3)
    dv = torch.empty_like(v).permute(0, 2, 1, 3)
    gpu.fa_bwd(qv, kv, vv, o, dov, lse, dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_fp64(qv.cpu(), kv.cpu(), vv.cpu(), dov.cpu(), True)
    check(dq, rq, "dQ")
    check(dk, rk, "dK")
    check(dv, rv, "dV")


def test_bwd_workspace_too_small(gpu):
    x = {n: torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16, device="cuda") for n in ("q", "k", "v", "o", "do")}
    lse = torch.zeros(1, 1, 8, device="cuda")
    ws = torch.empty(4, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_bwd(x["q"], x["k"], x["v"], x["o"], x["do"], lse, torch.empty_like(x["q"]),
                   torch.empty_like(x["k"]), torch.empty_like(x["v"]), workspace=ws)
    assert e.value.status == gpu.FA_ERR_WORKSPACE


def test_bwd_full_size(gpu):
    """The causal bf16 workload at full size (B=4, H=16, S=2048, d=128), in
    the launch configuration the benchmark times: every element of dQ, dK and
    dV against the oracle."""
    cfg = fa_inputs.CONFIGS["bf16_b4_h16_s2048_causal"]
    x = fa_inputs.make_fwd_inputs(cfg, seed=0, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(99)
    dout = torch.randn(cfg.B, cfg.Hq, cfg.Sq, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
    dq, dk, dv = run_bwd(gpu, x, dout, True)
    rq, rk, rv = oracle.attention_bwd_fp64(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), dout.cpu(), True)
    errs = [check(dq, rq, "dQ"), check(dk, rk, "dK"), check(dv, rv, "dV")]
    print("full-size backward, every element: relative max errors dQ/dK/dV", errs, flush=True)


@pytest.mark.timeout(900)
def test_bwd_long_context_full_size(gpu):
    """The long-context GQA backward at full size (Q [1, 32, 16384, 128], K/V
    [1, 8, 16384, 128], causal, 1 % outlier keys), with the inputs and launch
    the benchmark times: every element of dQ for the four query heads of one
    K/V head, and every element of that K/V head's dK and dV (the sum over
    its four query heads), against the oracle; and the two-role dK/dV
    schedule bit-identical to the default at this size."""
    cfg = fa_inputs.BWD_CONFIGS["bwd_bf16_gqa32x8_s16384_causal_outlier"]
    x = fa_inputs.make_bwd_inputs(cfg, seed=0, device="cuda")
    q, k, v, dout = x["q"], x["k"], x["v"], x["dout"]
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Sq, dtype=torch.float32, device="cuda")
    print("fa_fwd + fa_bwd, long-context GQA workload", flush=True)
    gpu.fa_fwd(q, k, v, o, lse, causal=True)
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    gpu.fa_bwd(q, k, v, o, dout, lse, *got, causal=True)
    pp = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    gpu.fa_bwd(q, k, v, o, dout, lse, *pp, causal=True, wave_pingpong=True)
    torch.cuda.synchronize()
    for name, u, w in zip(("dQ", "dK", "dV"), got, pp):
        assert torch.equal(u.view(torch.int16), w.view(torch.int16)), f"two-role schedule differs in {name}"
    G = cfg.Hq // cfg.Hkv
    kvh = 5
    heads = [(0, h) for h in range(G * kvh, G * kvh + G)]
    qc, kc, vc, dc = (t.cpu() for t in (q, k, v, dout))
    rq = rk = rv = None
    for bh in heads:  # one head at a time: each holds several S x S float64 arrays
        print(f"oracle backward, head {bh}", flush=True)
        hq, hk, hv = oracle.attention_bwd_fp64(qc, kc, vc, dc, True, heads=[bh])
        rq = hq if rq is None else rq + hq
        rk = hk if rk is None else rk + hk
        rv = hv if rv is None else rv + hv
        del hq, hk, hv
    h0, h1 = G * kvh, G * kvh + G
    errs = [check(got[0][:, h0:h1], rq[:, h0:h1], "dQ"),
            check(got[1][:, kvh:kvh + 1], rk[:, kvh:kvh + 1], "dK"),
            check(got[2][:, kvh:kvh + 1], rv[:, kvh:kvh + 1], "dV")]
    print("long-context backward, one K/V group, every element: relative max errors dQ/dK/dV", errs, flush=True)
