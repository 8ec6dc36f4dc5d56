"""GPU parity of fa_decode_kvq (int8 KV cache, split-KV + LSE combine; the
ragged-tail check also over an fp8 cache) against the float64 oracle fed the
same quantised cache."""

import dataclasses

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL_O = 8e-2   # quantised-KV path, against an oracle with the same quantisation
TOL_LSE = 1e-3


def run_decode(fa, x, num_splits, lse_wanted=True):
    B, Hq, d = x["q"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda") if lse_wanted else None
    print(f"fa_decode_kvq q={tuple(x['q'].shape)} cache={tuple(x['k'].shape)} splits={num_splits} "
          f"lens={x['seq_lens'].tolist()[:8]}", flush=True)
    fa.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse,
                     seq_lens=x["seq_lens"], num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def compare(o, lse, xc, heads=None):
    fmt = "int8" if xc["k"].dtype == torch.int8 else "fp8"
    ro, rl = oracle.decode_fp64(xc["q"], xc["k"].numpy(), xc["k_scale"].numpy(), xc["v"].numpy(),
                                xc["v_scale"].numpy(), xc["seq_lens"].numpy(), heads=heads, kv_format=fmt)
    og = o.double().cpu().numpy()
    sel = heads if heads is not None else [(b, h) for b in range(og.shape[0]) for h in range(og.shape[1])]
    bi = [b for b, _ in sel]
    hi = [h for _, h in sel]
    assert not np.isnan(og[bi, hi]).any()
    err_o = float(np.max(np.abs(og[bi, hi] - ro[bi, hi])))
    assert err_o <= TOL_O, f"O err {err_o}"
    if lse is not None:
        lg = lse.double().cpu().numpy()
        assert np.array_equal(np.isneginf(lg[bi, hi]), np.isneginf(rl[bi, hi]))
        fin = np.isfinite(rl[bi, hi])
        err_l = float(np.max(np.abs(lg[bi, hi][fin] - rl[bi, hi][fin]), initial=0.0))
        assert err_l <= TOL_LSE, f"LSE err {err_l}"
    return err_o


def make(B, Hq, Hkv, L, lens=None, seed=0):
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, 16, tuple(lens) if lens else ())
    xc = fa_inputs.make_decode_inputs(cfg, seed=seed)
    return xc, {k: v.cuda() for k, v in xc.items()}


CASES = [
    # B, Hq, Hkv, L, lens, splits
    (1, 4, 1, 1, None, 1),
    (2, 4, 1, 31, None, 3),
    (2, 8, 2, 100, [100, 37], 16),
    (3, 4, 4, 1000, [1000, 0, 513], 4),
    (2, 16, 1, 3000, [2999, 64], 16),
    (1, 32, 8, 4096, None, 16),
    (2, 2, 2, 700, [1, 699], 64),
]


@pytest.mark.parametrize("B,Hq,Hkv,L,lens,splits", CASES)
def test_decode_small(gpu, B, Hq, Hkv, L, lens, splits):
    xc, x = make(B, Hq, Hkv, L, lens, seed=L + Hq)
    o, lse = run_decode(gpu, x, splits)
    err = compare(o, lse, xc)
    print("max |dO|", err)


def test_decode_split_count_invariance(gpu):
    xc, x = make(2, 8, 2, 2048, [2048, 1500], seed=3)
    o1, l1 = run_decode(gpu, x, 1)
    o16, l16 = run_decode(gpu, x, 16)
    assert float((o1.float() - o16.float()).abs().max()) <= 1.6e-2
    assert float((l1 - l16).abs().max()) <= 1e-4


def test_decode_no_lse_and_deterministic(gpu):
    xc, x = make(2, 8, 2, 777, None, seed=4)
    o1, _ = run_decode(gpu, x, 5, lse_wanted=False)
    o2, _ = run_decode(gpu, x, 5, lse_wanted=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    compare(o1, None, xc)


def test_decode_workspace_too_small(gpu):
    xc, x = make(1, 4, 1, 64, None)
    o = torch.empty(1, 4, 128, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, None,
                          num_splits=4, workspace=ws)
    assert e.value.status == gpu.FA_ERR_WORKSPACE


def test_decode_full_size(gpu):
    """The int8 cache workload at full size (B=64, 32/8 heads, L=32768, 16
    splits), inputs drawn on the GPU, in the launch configuration the
    benchmark times; every (batch, head) row of O and LSE is compared with the
    oracle, and all of O is checked for unwritten (NaN) elements."""
    cfg = fa_inputs.CONFIGS["decode_int8_b64_gqa32x8_L32768"]
    x = fa_inputs.make_decode_inputs(cfg, seed=0, device="cuda")
    o, lse = run_decode(gpu, x, cfg.num_splits)
    assert not bool(torch.isnan(o.float()).any()) and not bool(torch.isnan(lse).any())
    xc = {k: v.cpu() for k, v in x.items()}
    del x
    err = compare(o, lse, xc)
    print(f"decode full size: every row, max|dO|={err:.3g}", flush=True)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("vec_scales", [True, False])
def test_decode_ragged_tail_tokens(gpu, fmt, vec_scales):
    """Every sequence length 1..40 and a few longer odd ones, with each query
    pointing at its sequence's LAST token so that this token dominates the
    softmax: a tail token lost, or read with a wrong scale, moves O and LSE far
    beyond the tolerance.  Both scale-load forms: 16-byte aligned scale rows
    (8-byte loads) and rows offset by one element (2-byte loads)."""
    lens = list(range(1, 41)) + [97, 255, 1001]
    B, Hq, Hkv, L = len(lens), 4, 1, 1024
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, 7, tuple(lens), fmt)
    xc = fa_inputs.make_decode_inputs(cfg, seed=17)
    deq = oracle.dequant_int8_fp64 if fmt == "int8" else oracle.dequant_fp8_fp64
    q = torch.empty(B, Hq, 128, dtype=torch.float64)
    for b, n in enumerate(lens):
        last = deq(xc["k"][b, 0, n - 1:n].numpy(), xc["k_scale"][b, 0, n - 1:n].numpy())[0]
        for h in range(Hq):
            q[b, h] = torch.from_numpy(last * (3.0 + h) / max(1e-9, float(np.abs(last).max())))
    xc["q"] = q.to(torch.bfloat16)
    x = {k: v.cuda() for k, v in xc.items()}
    if not vec_scales:  # the same scales one element into a larger buffer: 2-byte aligned rows
        for key in ("k_scale", "v_scale"):
            big = torch.zeros(B, Hkv, L + 1, dtype=torch.float16, device="cuda")
            big[..., 1:] = x[key]
            x[key] = big[..., 1:]
    o, lse = run_decode(gpu, x, 7)
    compare(o, lse, xc)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_decode_value_scales_spanning_the_chunk(gpu, fmt):
    """Value scales 4096 times larger on one 32-token tile of a split, which a
    wavefront other than the one scanning that stretch of scales consumes: the
    fp16 prescale of P * v_scale must cover the whole chunk, or that tile's
    weights overflow.  The query points at one of those tokens, so they carry
    most of the probability.  Compared relative to the output's magnitude
    (the dequantised values reach about 1e4 here)."""
    B, Hq, Hkv, L, splits = 1, 4, 1, 1024, 4   # chunks of 256 tokens: 8 tiles, two per wavefront
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, splits, (), fmt)
    xc = fa_inputs.make_decode_inputs(cfg, seed=23)
    for s in range(splits):   # tile 5 of every chunk
        lo = s * 256 + 5 * 32
        xc["v_scale"][0, 0, lo:lo + 32] = (xc["v_scale"][0, 0, lo:lo + 32].float() * 4096).half()
    deq = oracle.dequant_int8_fp64 if fmt == "int8" else oracle.dequant_fp8_fp64
    tok = 2 * 256 + 5 * 32 + 7
    key = deq(xc["k"][0, 0, tok:tok + 1].numpy(), xc["k_scale"][0, 0, tok:tok + 1].numpy())[0]
    for h in range(Hq):
        xc["q"][0, h] = torch.from_numpy(key * (1.0 + h) / float(np.abs(key).max())).to(torch.bfloat16)
    x = {k: v.cuda() for k, v in xc.items()}
    o, lse = run_decode(gpu, x, splits)
    ro, rl = oracle.decode_fp64(xc["q"], xc["k"].numpy(), xc["k_scale"].numpy(), xc["v"].numpy(),
                                xc["v_scale"].numpy(), xc["seq_lens"].numpy(), kv_format=fmt)
    og = o.double().cpu().numpy()
    assert np.isfinite(og).all()
    scale = float(np.abs(ro).max())
    assert scale > 100.0   # the large-scale tokens dominate
    err = float(np.max(np.abs(og - ro))) / scale
    assert err <= 1e-2, f"relative O err {err}"
    assert float(np.max(np.abs(lse.double().cpu().numpy() - rl))) <= TOL_LSE


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("path", ["staged", "staged2", "vec8", "scalar2"])
def test_decode_poisoned_cache_tail(gpu, fmt, path):
    """Cache slots at or past seq_lens[b] hold +-Inf and NaN fp16 scales
    (0x7C00, 0xFC00, 0x7E00) and, for fp8, the NaN codes 0x7F / 0xFF: only
    the first seq_lens[b] tokens may reach the result.  Lengths are not
    multiples of 32 or 4.  The four scale paths: scales staged in LDS (chunks
    of at most 2048 tokens) with 16-byte loads or, for scale rows offset by
    one element, 2-byte loads; per-tile 8-byte scale loads (longer chunks);
    per-tile 2-byte loads (longer chunks, offset rows)."""
    lens = [184, 1, 3001, 2047, 33, 4095]
    B, Hq, Hkv, L = len(lens), 8, 2, 4096
    splits = 4 if path.startswith("staged") else 1  # chunks of 1024 or 4096 tokens
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, splits, tuple(lens), fmt)
    xc = fa_inputs.make_decode_inputs(cfg, seed=31)
    x = {k: v.clone() for k, v in xc.items()}
    bits = torch.tensor([0x7C00, 0xFC00, 0x7E00], dtype=torch.int32).to(torch.int16)
    for b, n in enumerate(lens):
        pat = bits[torch.arange(L - n) % 3].view(torch.float16)
        for key in ("k_scale", "v_scale"):
            x[key][b, :, n:] = pat
        for key in ("k", "v"):
            if fmt == "fp8":
                x[key][b, :, n:] = torch.where(torch.arange(L - n)[:, None] % 2 == 0, 0x7F, 0xFF).to(torch.uint8)
            else:
                x[key][b, :, n:] = 127
    x = {k: v.cuda() for k, v in x.items()}
    if path in ("scalar2", "staged2"):
        for key in ("k_scale", "v_scale"):
            big = torch.zeros(B, Hkv, L + 1, dtype=torch.float16, device="cuda")
            big[..., 1:] = x[key]
            x[key] = big[..., 1:]
    o, lse = run_decode(gpu, x, splits)
    assert bool(torch.isfinite(o.float()).all()), "a token past seq_lens reached the output"
    compare(o, lse, xc)
