"""GPU parity of the fp8 accuracy variants:

* fa_fp8_quantize (64-row block scales, optional random-sign Hadamard rotation)
  against the oracle's quantiser: codes and scales bit-exact;
* fa_fwd on fp8 codes with block descales against the float64 oracle fed the
  same dequantised values (O within 8e-2, LSE within 1e-3), with the
  probabilities rounded to e4m3 or (fp8_p_bf16) to bf16 for P V;
* the variants' error against exact attention of the unquantised bf16 inputs
  on the long-context workload's outlier distribution (1 % of key rows x 8),
  per-tensor scales versus block scales versus block scales with rotation.
"""

import dataclasses

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL_O = 8e-2
TOL_LSE = 1e-3
# The fp8 matrix instructions sum their products to about 2^-11.4 of the
# largest product (measured by test_fp8_score_accumulation_precision through
# the LSE of a single-key problem); a score of d = 128 takes two 64-deep
# instructions, so its error is at most 2^-10 of its largest product.
FP8_ACC_REL = 2.0 ** -10


def fp8_lse_bound(qd, kd, causal, G, tau):
    """Per-row bound on the fp8 path's LSE error from the score accumulation:
    the LSE moves by at most the largest score error among the visible keys,
    FP8_ACC_REL * tau * max over visible keys j and channels c of
    |q_ic k_jc| (dequantised values); at least the 1e-3 bar.  [B, Hq, Sq]."""
    B, Hq, Sq, d = qd.shape
    Sk = kd.shape[2]
    out = np.empty((B, Hq, Sq))
    for b in range(B):
        for kh in range(kd.shape[1]):
            ak = np.abs(kd[b, kh])
            vis = np.maximum.accumulate(ak, axis=0) if causal else np.broadcast_to(ak.max(axis=0), ak.shape)
            rows = np.minimum(np.arange(Sq) + Sk - Sq, Sk - 1).clip(0)
            for h in range(kh * G, kh * G + G):
                out[b, h] = np.max(np.abs(qd[b, h]) * vis[rows], axis=1)
    return np.maximum(TOL_LSE, FP8_ACC_REL * tau * out)


def _signs(seed, d=128):
    g = torch.Generator().manual_seed(seed)
    return torch.where(torch.rand(d, generator=g) < 0.5, -1.0, 1.0).to(torch.float32)


def gpu_quant(fa, x, signs=None):
    B, H, S, d = x.shape
    codes = torch.full((B, H, S, d), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, H, (S + 63) // 64), float("nan"), dtype=torch.float32, device="cuda")
    print(f"fa_fp8_quantize x={tuple(x.shape)} {x.dtype} rotate={signs is not None}", flush=True)
    fa.fa_fp8_quantize(x.cuda(), codes, scales, None if signs is None else signs.cuda())
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu()


QUANT_CASES = [
    # B, H, S, dtype, rotate
    (1, 1, 1, torch.bfloat16, False),
    (2, 3, 150, torch.bfloat16, False),
    (2, 3, 150, torch.bfloat16, True),
    (1, 2, 64, torch.float16, True),
    (1, 2, 333, torch.float16, False),
]


@pytest.mark.parametrize("B,H,S,dt,rot", QUANT_CASES)
def test_quantise_bit_exact(gpu, B, H, S, dt, rot):
    g = torch.Generator().manual_seed(S + H)
    x = torch.randn(B, H, S, 128, generator=g)
    if S > 100:
        x[0, 0, 70] *= 8.0  # an outlier row
        x[0, H - 1, 64:128] = 0.0  # an all-zero block
        x[B - 1, 0, 3, 9] = 300.0  # an outlier channel entry
        x[B - 1, 0, 5] *= 1e-6  # tiny values (subnormal codes)
    x = x.to(dt)
    signs = _signs(S) if rot else None
    codes, scales = gpu_quant(gpu, x, signs)
    rc, rs = oracle.quantize_fp8_blocks(x, None if signs is None else signs.numpy())
    assert np.array_equal(scales.numpy().view(np.uint32), rs.view(np.uint32))
    bad = np.argwhere(codes.numpy() != rc)
    assert len(bad) == 0, f"codes differ at {bad[:5].tolist()} (of {len(bad)})"


def _fp8_inputs(cfg, seed, signs=None, block=True):
    """bf16 draws of the configuration, quantised by the oracle; returns the GPU
    tensors and the dequantised float64 values."""
    x = fa_inputs.make_fwd_inputs(dataclasses.replace(cfg, dtype="bf16", out_dtype=""), seed=seed)
    out, deq = {}, {}
    for n in ("q", "k", "v"):
        s = signs if n in ("q", "k") else None
        if block:
            c, sc = oracle.quantize_fp8_blocks(x[n], s)
            out[n], out[n + "_bs"] = torch.from_numpy(c), torch.from_numpy(sc)
            deq[n] = oracle.dequant_fp8_blocks_fp64(c, sc)
        else:
            xf = x[n].float()
            if s is not None:
                xf = torch.from_numpy(oracle.hadamard_rotate_fp32(xf.numpy(), s))
            c8, ts = fa_inputs.quantize_fp8_per_tensor(xf)
            out[n], out[n + "_ts"] = c8.view(torch.uint8), ts
            deq[n] = oracle.e4m3_decode(c8.view(torch.uint8)) * ts
    return x, out, deq


def run_fp8(fa, out, causal, block=True, p_bf16=False):
    q, k, v = (out[n].cuda().view(torch.float8_e4m3fn) for n in ("q", "k", "v"))
    B, Hq, Sq, d = q.shape
    o = torch.full((B, Hq, Sq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    print(f"fa_fwd fp8 q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} block={block} p_bf16={p_bf16}",
          flush=True)
    if block:
        bds = tuple(out[n + "_bs"].cuda().contiguous() for n in ("q", "k", "v"))
        fa.fa_fwd(q, k, v, o, lse, causal=causal, block_descales=bds, p_bf16=p_bf16)
    else:
        fa.fa_fwd(q, k, v, o, lse, causal=causal, q_descale=out["q_ts"], k_descale=out["k_ts"],
                  v_descale=out["v_ts"], p_bf16=p_bf16)
    torch.cuda.synchronize()
    return o, lse


FWD_CASES = [
    # B, Hq, Hkv, Sq, Sk, causal
    (1, 2, 2, 64, 64, False),
    (2, 4, 2, 200, 200, True),
    (1, 4, 1, 130, 333, False),
    (1, 2, 2, 300, 129, True),
    (1, 8, 8, 512, 512, True),
]


@pytest.mark.parametrize("p_bf16", [False, True], ids=["p_e4m3", "p_bf16"])
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", FWD_CASES)
def test_block_descale_forward(gpu, B, Hq, Hkv, Sq, Sk, causal, p_bf16):
    # the fp8 workload's distribution (N(0,1) draws, no outlier rows)
    cfg = fa_inputs.FwdConfig("t", "fp8", B, Hq, Hkv, Sq, Sk, 128, causal)
    _, out, deq = _fp8_inputs(cfg, seed=Sq + Sk)
    o, lse = run_fp8(gpu, out, causal, p_bf16=p_bf16)
    ro, rl = oracle.attention_fp64(deq["q"], deq["k"], deq["v"], causal)
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert not np.isnan(og).any()
    assert float(np.max(np.abs(og - ro))) <= TOL_O
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lg), fin)
    assert float(np.max(np.abs(lg[fin] - rl[fin]))) <= TOL_LSE


def _variant_errors(fa, cfg, channel_outlier=False, seed=11):
    """max |O - exact| and max |LSE - exact| of per-tensor, block and
    block + rotation fp8 attention, exact = the float64 oracle on the bf16
    inputs before quantisation."""
    signs = _signs(5).numpy()
    base = fa_inputs.make_fwd_inputs(dataclasses.replace(cfg, dtype="bf16", out_dtype=""), seed=seed)
    if channel_outlier:  # the alternative reading: one key channel x 8 in every row
        base["k"] = (base["k"].float() * torch.where(torch.arange(128) == 5, 8.0, 1.0)).to(torch.bfloat16)
    ro, rl = oracle.attention_fp64(base["q"], base["k"], base["v"], cfg.causal)
    errs = {}
    for name, block, sg in (("per-tensor", False, None), ("block", True, None), ("block+rotation", True, signs)):
        out = {}
        for n in ("q", "k", "v"):
            s = sg if n in ("q", "k") else None
            if block:
                c, sc = oracle.quantize_fp8_blocks(base[n], s)
                out[n], out[n + "_bs"] = torch.from_numpy(c), torch.from_numpy(sc)
            else:
                c8, ts = fa_inputs.quantize_fp8_per_tensor(base[n].float())
                out[n], out[n + "_ts"] = c8.view(torch.uint8), ts
        o, lse = run_fp8(fa, out, cfg.causal, block=block)
        errs[name] = (float(np.max(np.abs(o.double().cpu().numpy() - ro))),
                      float(np.max(np.abs(lse.double().cpu().numpy() - rl))))
    return errs


def test_variants_against_exact_on_outliers(gpu):
    """fp8 error against exact attention of the unquantised bf16 inputs, GQA 4/1,
    causal, S = 1024, for the long-context workload's outliers read two ways:
    1 % of key rows x 8 (the reading the workload uses), where block scales cut
    the error of per-tensor scales; and one key channel x 8, where the rotation
    cuts it further.  Against exact attention the quantisation error of Q, K
    and V adds to the kernel's own, so these errors exceed the 8e-2 bar, which
    is stated against an oracle fed the same codes; they are printed for the
    record."""
    cfg = fa_inputs.FwdConfig("t", "fp8", 1, 4, 1, 1024, 1024, 128, True, outlier_frac=0.01)
    rows = _variant_errors(gpu, cfg)
    chan = _variant_errors(gpu, dataclasses.replace(cfg, outlier_frac=0.0), channel_outlier=True)
    print("row outliers: max |O - exact|, max |LSE - exact|:", rows)
    print("channel outlier: max |O - exact|, max |LSE - exact|:", chan)
    assert rows["block"][0] < rows["per-tensor"][0]
    assert chan["block+rotation"][0] < chan["block"][0]


def test_quantise_then_forward_full_size(gpu):
    """The fp8 workload's shape (B=8, H=16, S=4096) quantised on the GPU with
    block scales and rotation, then the block-descale forward, as the
    benchmark's block-scaled workload runs it: every code and scale of Q, K
    and V bit-exact against the oracle's quantiser (the quantiser workload's
    full size), and every element of O and LSE against the oracle on the
    dequantised codes."""
    cfg = fa_inputs.CONFIGS["fp8_b8_h16_s4096"]
    x = fa_inputs.make_fwd_inputs(dataclasses.replace(cfg, dtype="bf16", out_dtype=""), seed=0, device="cuda")
    signs = _signs(7).cuda()
    out = {}
    for n in ("q", "k", "v"):
        t = x[n]
        codes = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
        sc = torch.empty(t.shape[0], t.shape[1], t.shape[2] // 64, dtype=torch.float32, device="cuda")
        gpu.fa_fp8_quantize(t, codes, sc, signs if n != "v" else None)
        out[n], out[n + "_bs"] = codes, sc
    o, lse = run_fp8(gpu, out, False)
    for n in ("q", "k", "v"):
        print(f"oracle quantiser, {n}", flush=True)
        rc, rs = oracle.quantize_fp8_blocks(x[n].cpu(), signs.cpu().numpy() if n != "v" else None)
        assert np.array_equal(out[n + "_bs"].cpu().numpy().view(np.uint32), rs.view(np.uint32)), n
        assert np.array_equal(out[n].cpu().numpy(), rc), n
        del rc, rs
    deq = {n: oracle.dequant_fp8_blocks_fp64(out[n].cpu().numpy(), out[n + "_bs"].cpu().numpy())
           for n in ("q", "k", "v")}
    print("oracle forward, every head", flush=True)
    ro, rl = oracle.attention_fp64(deq["q"], deq["k"], deq["v"], False)
    err_o = float(np.max(np.abs(o.double().cpu().numpy() - ro)))
    err_l = float(np.max(np.abs(lse.double().cpu().numpy() - rl)))
    print(f"block-scaled, rotated fp8 at full size, every element: max|dO|={err_o:.3g} max|dLSE|={err_l:.3g}")
    assert err_o <= TOL_O and err_l <= TOL_LSE


def test_block_descales_of_any_ratio(gpu):
    """Block descales that are not powers of two (plain absmax / 448 per
    64-row block, and V blocks whose absmax differs by factors up to ~40 so the
    descale ratios are arbitrary): the V ratio is folded into the
    probabilities before their rounding, which with bf16 probabilities adds no
    error beyond that rounding.  Every element within the 8e-2 bar with bf16
    probabilities; the e4m3 mode is held to its documented envelope,
    2^-4 max|V| (+1e-2), since the V blocks here reach |V| of about 16."""
    B, Hq, Hkv, S = 1, 4, 2, 700
    g = torch.Generator().manual_seed(41)
    raw = {n: torch.randn(B, Hq if n == "q" else Hkv, S, 128, generator=g) for n in ("q", "k", "v")}
    raw["v"] *= torch.exp(torch.randn(B, Hkv, S // 64 + 1, 1, generator=g)).repeat_interleave(64, 2)[:, :, :S]
    out, deq = {}, {}
    for n, t in raw.items():
        t = t.to(torch.bfloat16).float()
        nb = (S + 63) // 64
        pad = torch.zeros(B, t.shape[1], nb * 64, 128)
        pad[:, :, :S] = t
        amax = pad.view(B, t.shape[1], nb, 64 * 128).abs().amax(-1)
        sc = (amax / 448.0).to(torch.float32)
        y = (pad / sc.repeat_interleave(64, 2)[..., None]).clamp(-448, 448)[:, :, :S]
        out[n] = y.to(torch.float8_e4m3fn).view(torch.uint8)
        out[n + "_bs"] = sc.contiguous()
        deq[n] = oracle.dequant_fp8_blocks_fp64(out[n].numpy(), sc.numpy())
    assert not bool(torch.frexp(out["v_bs"]).mantissa.eq(0.5).all())  # not powers of two
    ro, rl = oracle.attention_fp64(deq["q"], deq["k"], deq["v"], True)
    vmax = float(np.max(np.abs(deq["v"])))
    for p_bf16 in (True, False):
        o, lse = run_fp8(gpu, out, True, p_bf16=p_bf16)
        err = float(np.max(np.abs(o.double().cpu().numpy() - ro)))
        print(f"non-power-of-two block descales, p_bf16={p_bf16}: max|dO|={err:.3g} (max|V| {vmax:.3g})")
        assert err <= (TOL_O if p_bf16 else 2.0 ** -4 * vmax + 1e-2)
        assert float(np.max(np.abs(lse.double().cpu().numpy() - rl))) <= TOL_LSE


def test_fp8_score_accumulation_precision(gpu):
    """The fp8 path's score precision, measured through the public call: with a
    single key, LSE = softmax_scale * (q . k) exactly, so LSE against the exact
    float64 dot product of the codes shows how precisely the fp8 matrix core
    sums its 128 products.  bf16 inputs (exactly the same values, the same
    call) sum to fp32 precision; fp8 inputs to about 2^-11.4 of the largest
    product per 64-deep instruction.  The test pins that ratio below the
    2^-10 the fp8 LSE bound above relies on, and prints it."""
    S = 4096
    g = torch.Generator().manual_seed(3)
    c = torch.randint(0, 256, (2, S, 128), generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    q8 = c[0].view(1, 1, S, 128).contiguous()
    k8 = c[1, :1].view(1, 1, 1, 128).contiguous()
    qf, kf = oracle.e4m3_decode(q8.numpy()), oracle.e4m3_decode(k8.numpy())
    exact = (qf[0, 0] @ kf[0, 0, 0])                         # [S]
    pmax = np.max(np.abs(qf[0, 0] * kf[0, 0, 0]), axis=1)   # largest product per row
    res = {}
    for name in ("fp8", "bf16"):
        if name == "fp8":
            q, k = q8.cuda().view(torch.float8_e4m3fn), k8.cuda().view(torch.float8_e4m3fn)
            o = torch.empty(1, 1, S, 128, dtype=torch.bfloat16, device="cuda")
        else:  # the same values in bf16 (every e4m3 value is a bf16 value)
            q = torch.from_numpy(qf).to(torch.bfloat16).cuda()
            k = torch.from_numpy(kf).to(torch.bfloat16).cuda()
            o = torch.empty_like(q)
        lse = torch.empty(1, 1, S, device="cuda")
        print(f"fa_fwd {name} single key, {S} rows", flush=True)
        gpu.fa_fwd(q, k, k, o, lse, causal=False, softmax_scale=1.0)
        torch.cuda.synchronize()
        err = np.abs(lse[0, 0].double().cpu().numpy() - exact) / np.maximum(pmax, 1e-30)
        res[name] = float(err.max())
    print("max |LSE - q.k| / max|product|: fp8 2^%.1f, bf16 2^%.1f"
          % (np.log2(max(res["fp8"], 1e-30)), np.log2(max(res["bf16"], 1e-30))))
    assert res["fp8"] <= FP8_ACC_REL
    assert res["bf16"] <= 2.0 ** -18


@pytest.mark.timeout(900)
def test_variants_on_the_long_context_outlier_workload(gpu):
    """The fp8 variants at the long-context workload's full shape and outlier
    distribution (Q [1, 32, 16384, 128], K/V [1, 8, 16384, 128], 164 key rows
    per kv head x 8, causal), quantised on the GPU: per-tensor scales, 64-row
    block scales, block scales with rotation; every element of O and LSE
    against the oracle fed the variant's own codes.

    With bf16 probabilities (fp8_p_bf16) every variant meets the fp8 bar,
    8e-2.  With e4m3 probabilities it cannot be promised here: the outlier
    keys concentrate the softmax on a few keys, and e4m3 keeps 3 mantissa
    bits, so a probability carries up to 2^-4 of itself as rounding and one
    output element moves by up to about 2^-4 * max |V| (plus the far smaller
    absolute rounding of probabilities in the subnormal range).  That mode is
    held to this documented envelope (+1e-2), a mean error of 1e-2, and the
    1e-3 LSE bar, which the rounding of P does not touch.  The error of each
    variant against exact attention of the bf16 inputs is printed on sampled
    heads and rows, for the record.

    LSE: the 1e-3 bar where the fp8 score accumulation allows it, else the
    per-row bound fp8_lse_bound derives from it.  Outlier keys make scores of
    30-50, and the fp8 matrix instructions sum products to about 2^-11.4 of
    the largest one (test_fp8_score_accumulation_precision), so the LSE of
    rows dominated by outlier keys moves by up to ~2e-3 (measured 1.6e-3);
    every row is held to its bound."""
    cfg = fa_inputs.CONFIGS["bf16_gqa32x8_s16384_causal_outlier"]
    x = fa_inputs.make_fwd_inputs(cfg, seed=0, device="cuda")
    signs = fa_inputs.make_rotation_signs(128, seed=0, device="cuda")
    heads = [0, 13, 31]
    rows = [0, 1, 4095, 8192, 16383]
    exact = oracle.attention_fp64(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True, rows=rows,
                                  heads=[(0, h) for h in heads])
    report = {}
    for name in ("per-tensor", "block", "block+rotation"):
        out = {}
        if name == "per-tensor":
            for n in ("q", "k", "v"):
                c8, ts = fa_inputs.quantize_fp8_per_tensor(x[n])
                out[n], out[n + "_ts"] = c8.view(torch.uint8), ts
            deq = {n: oracle.e4m3_decode(out[n].cpu().numpy()) * out[n + "_ts"] for n in ("q", "k", "v")}
        else:
            for n in ("q", "k", "v"):
                t = x[n]
                codes = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
                sc = torch.empty(t.shape[0], t.shape[1], t.shape[2] // 64, dtype=torch.float32, device="cuda")
                rot = signs if (name == "block+rotation" and n != "v") else None
                gpu.fa_fp8_quantize(t, codes, sc, rot)
                out[n], out[n + "_bs"] = codes, sc
            deq = {n: oracle.dequant_fp8_blocks_fp64(out[n].cpu().numpy(), out[n + "_bs"].cpu().numpy())
                   for n in ("q", "k", "v")}
        ro, rl = oracle.attention_fp64(deq["q"], deq["k"], deq["v"], True)
        vmax = float(np.max(np.abs(deq["v"])))
        lse_bar = fp8_lse_bound(deq["q"], deq["k"], True, 4, cfg.scale)
        del deq
        for p_bf16 in (True, False):
            o, lse = run_fp8(gpu, out, True, block=name != "per-tensor", p_bf16=p_bf16)
            og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
            d = np.abs(og - ro)
            dl = np.abs(lg - rl)
            par = (float(d.max()), float(d.mean()), float(dl.max()))
            over = int((dl > TOL_LSE).sum())
            ex = (float(np.max(np.abs(og[:, heads][:, :, rows] - exact[0][:, heads]))),
                  float(np.max(np.abs(lg[:, heads][:, :, rows] - exact[1][:, heads]))))
            mode = "p_bf16" if p_bf16 else "p_e4m3"
            report[f"{name}/{mode}"] = {"parity_max_mean_lse": par, "vs_exact_sampled": ex}
            print(f"{name} {mode}: every element, max|dO|={par[0]:.3g} mean|dO|={par[1]:.3g} "
                  f"max|dLSE|={par[2]:.3g} ({over} rows above 1e-3, largest bound {lse_bar.max():.3g}); "
                  f"vs exact (sampled) {ex[0]:.3g}, {ex[1]:.3g}", flush=True)
            assert bool(np.all(dl <= lse_bar)), (name, mode, par)
            if p_bf16:
                assert par[0] <= TOL_O, (name, mode, par)
            else:
                assert par[0] <= 2.0 ** -4 * vmax + 1e-2 and par[1] <= 1e-2, (name, mode, par)
            del o, lse
        del out
    print("long-context outliers, full shape, every element:", report)
