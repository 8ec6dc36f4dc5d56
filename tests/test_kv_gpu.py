"""GPU parity of the cache's other formats and its write side:

* fa_kv_append (quantise-on-append, int8 and E4M3FN, bf16 and fp16 rows) against
  the oracle's quantiser: codes and scales bit-exact, untouched slots unchanged;
* fa_decode_kvq over an E4M3FN cache, and with a bf16 residual window, against
  the float64 oracle fed the same cache (O within 8e-2, LSE within 1e-3);
* append then decode, end to end.
"""

import numpy as np
import pytest
import torch

import fa_inputs
import oracle
from kv_boundary import boundary_rows

pytestmark = pytest.mark.gpu

TOL_O = 8e-2
TOL_LSE = 1e-3
SENTINEL = 0x5A


# ---- quantise-on-append -----------------------------------------------------------

def _append_case(B, H, T, L, pos, fmt, in_dtype, seed):
    g = torch.Generator().manual_seed(seed)
    kn = torch.randn(B, H, T, 128, generator=g)
    vn = torch.randn(B, H, T, 128, generator=g)
    # rows that stress the quantiser: all zero, large, tiny (scale underflows
    # fp16), one with exact half-step ties, a single spike
    if T >= 6:
        kn[0, 0, 0] = 0
        vn[0, 0, 1] *= 3000
        kn[0, 0, 2] *= 1e-9
        kn[0, 0, 3] = 0
        kn[0, 0, 3, 0] = 127 / 16
        kn[0, 0, 3, 1:5] = torch.tensor([0.5, 1.5, 2.5, -0.5]) / 16
        vn[0, 0, 4] = 0
        vn[0, 0, 4, 77] = -5.0
        kn[0, 0, 5, :64] = -kn[0, 0, 5, :64].abs()
    kn, vn = kn.to(in_dtype), vn.to(in_dtype)
    cdt = torch.int8 if fmt == "int8" else torch.uint8
    kc = torch.full((B, H, L, 128), SENTINEL, dtype=cdt)
    vc = torch.full((B, H, L, 128), SENTINEL, dtype=cdt)
    ks = torch.full((B, H, L), 7.0, dtype=torch.float16)
    vs = torch.full((B, H, L), 7.0, dtype=torch.float16)
    positions = torch.tensor(pos, dtype=torch.int32)
    return {"k_new": kn, "v_new": vn, "k_cache": kc, "v_cache": vc, "k_scale": ks, "v_scale": vs,
            "positions": positions}


def _run_append(fa, xc, fmt, with_positions=True):
    x = {k: v.cuda() for k, v in xc.items()}
    print(f"fa_kv_append fmt={fmt} rows={tuple(x['k_new'].shape)} dtype={x['k_new'].dtype} "
          f"cache={tuple(x['k_cache'].shape)} pos={xc['positions'].tolist()[:8]}", flush=True)
    fa.fa_kv_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                    positions=x["positions"] if with_positions else None)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in x.items()}


def _check_append(out, xc, fmt, with_positions=True):
    pos = xc["positions"].numpy() if with_positions else None
    for side in ("k", "v"):
        rc, rs = oracle.kv_append_ref(xc[f"{side}_cache"].numpy(), xc[f"{side}_scale"].numpy(),
                                      xc[f"{side}_new"], pos, fmt)
        gc = out[f"{side}_cache"].numpy()
        gs = out[f"{side}_scale"].numpy()
        bad = np.argwhere(gc.view(np.uint8) != rc.view(np.uint8))
        assert len(bad) == 0, f"{side} codes differ at {bad[:5].tolist()} (of {len(bad)})"
        assert np.array_equal(gs.view(np.uint16), rs.view(np.uint16)), f"{side} scales differ"


APPEND_CASES = [
    # B, H, T, L, positions
    (1, 1, 1, 8, [3]),
    (2, 3, 37, 64, [0, 40]),      # the second sequence runs past the end: 13 rows dropped
    (3, 2, 50, 64, [-5, 14, 64]),  # leading rows dropped; a sequence wholly past the end
    (2, 8, 300, 512, [100, 212]),
]


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("B,H,T,L,pos", APPEND_CASES)
def test_append_bit_exact(gpu, fmt, in_dtype, B, H, T, L, pos):
    xc = _append_case(B, H, T, L, pos, fmt, in_dtype, seed=T + L)
    out = _run_append(gpu, xc, fmt)
    _check_append(out, xc, fmt)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float16])
def test_append_codes_at_rounding_boundaries(gpu, fmt, in_dtype):
    """Every entry on, or one or two input-type ulps from, a rounding boundary
    of its code (and the clamp at QMAX): codes and scales bit-exact against the
    oracle's correctly rounded float32 quotient."""
    n = 4096
    k = boundary_rows(fmt, in_dtype, n, seed=31).reshape(1, 2, n // 2, 128)
    v = boundary_rows(fmt, in_dtype, n, seed=32).reshape(1, 2, n // 2, 128)
    cdt = torch.int8 if fmt == "int8" else torch.uint8
    L = n // 2
    xc = {"k_new": k, "v_new": v,
          "k_cache": torch.full((1, 2, L, 128), SENTINEL, dtype=cdt),
          "v_cache": torch.full((1, 2, L, 128), SENTINEL, dtype=cdt),
          "k_scale": torch.full((1, 2, L), 7.0, dtype=torch.float16),
          "v_scale": torch.full((1, 2, L), 7.0, dtype=torch.float16),
          "positions": torch.tensor([0], dtype=torch.int32)}
    out = _run_append(gpu, xc, fmt)
    _check_append(out, xc, fmt)


def test_append_without_positions_starts_at_zero(gpu):
    xc = _append_case(2, 2, 20, 32, [0, 0], "fp8", torch.bfloat16, seed=5)
    out = _run_append(gpu, xc, "fp8", with_positions=False)
    _check_append(out, xc, "fp8", with_positions=False)


def test_append_strided_views(gpu):
    # rows taken from a [B, T, H, d] (token-major) buffer, cache inside a larger one
    g = torch.Generator().manual_seed(9)
    base_k = torch.randn(2, 24, 4, 128, generator=g).to(torch.bfloat16)
    base_v = torch.randn(2, 24, 4, 128, generator=g).to(torch.bfloat16)
    kn, vn = base_k.permute(0, 2, 1, 3), base_v.permute(0, 2, 1, 3)
    big_k = torch.full((2, 4, 80, 144), SENTINEL, dtype=torch.int8)
    big_v = torch.full((2, 4, 80, 144), SENTINEL, dtype=torch.int8)
    ks = torch.full((2, 4, 80), 7.0, dtype=torch.float16)
    vs = torch.full((2, 4, 80), 7.0, dtype=torch.float16)
    x = {"kn": kn.cuda(), "vn": vn.cuda(), "bk": big_k.cuda(), "bv": big_v.cuda(), "ks": ks.cuda(), "vs": vs.cuda()}
    pos = torch.tensor([5, 60], dtype=torch.int32, device="cuda")
    print("fa_kv_append strided views", flush=True)
    gpu.fa_kv_append(x["kn"], x["vn"], x["bk"][..., :128], x["bv"][..., :128], x["ks"], x["vs"], positions=pos)
    torch.cuda.synchronize()
    for side, new, big, sc in (("k", kn, x["bk"], x["ks"]), ("v", vn, x["bv"], x["vs"])):
        rc, rs = oracle.kv_append_ref(np.full((2, 4, 80, 128), SENTINEL, dtype=np.int8),
                                      np.full((2, 4, 80), 7.0, dtype=np.float16),
                                      new.contiguous(), pos.cpu().numpy(), "int8")
        got = big.cpu()
        assert np.array_equal(got[..., :128].numpy(), rc)
        assert np.all(got[..., 128:].numpy() == SENTINEL)  # padding columns untouched
        assert np.array_equal(sc.cpu().numpy().view(np.uint16), rs.view(np.uint16))


def test_append_full_size(gpu):
    """The 4096-token append workload at full size (64 sequences x 8 heads into
    32768-slot caches at position 28672), in the launch the benchmark times:
    every code and scale of every (batch, head) slice bit-exact against the
    oracle, and every slot outside the chunk still zero."""
    for name in ("append_int8_b64_h8_t4096", "append_fp8_b64_h8_t4096"):
        cfg = fa_inputs.KV_CONFIGS[name]
        x = fa_inputs.make_append_inputs(cfg, seed=0, device="cuda")
        print(f"fa_kv_append {name}", flush=True)
        gpu.fa_kv_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                         positions=x["positions"])
        torch.cuda.synchronize()
        p0, p1 = cfg.pos0, cfg.pos0 + cfg.T
        for side in ("k", "v"):
            print(f"oracle quantiser, {name} {side}", flush=True)
            rc, rs = oracle.quantize_kv_tokhead(x[f"{side}_new"].cpu(), cfg.kv_format)
            gc = x[f"{side}_cache"][:, :, p0:p1].cpu().numpy()
            gs = x[f"{side}_scale"][:, :, p0:p1].cpu().numpy()
            assert np.array_equal(gc.view(np.uint8), rc.view(np.uint8))
            assert np.array_equal(gs.view(np.uint16), rs.view(np.uint16))
            del rc, rs, gc, gs
            cache, sc = x[f"{side}_cache"], x[f"{side}_scale"]
            raw = cache.view(torch.uint8)
            assert not bool(raw[:, :, :p0].ne(0).any()) and not bool(raw[:, :, p1:].ne(0).any())
            assert not bool(sc[:, :, :p0].ne(0).any()) and not bool(sc[:, :, p1:].ne(0).any())
        del x
        torch.cuda.empty_cache()


# ---- fp8-KV and residual-window decode ------------------------------------------------

def _decode(fa, x, num_splits, window):
    B, Hq, d = x["q"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    kw = {}
    if window:
        kw = {"k_recent": x["k_recent"], "v_recent": x["v_recent"], "recent_lens": x["recent_lens"]}
    print(f"fa_decode_kvq cache={tuple(x['k'].shape)} {x['k'].dtype} splits={num_splits} "
          f"lens={x['seq_lens'].tolist()[:8]} window={tuple(x['k_recent'].shape) if window else None} "
          f"recent={x['recent_lens'].tolist()[:8] if window else None}", flush=True)
    fa.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse,
                     seq_lens=x["seq_lens"], num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return o, lse


def _compare(o, lse, xc, fmt, window, heads=None):
    kw = {}
    if window:
        kw = {"k_recent": xc["k_recent"], "v_recent": xc["v_recent"], "recent_lens": xc["recent_lens"].numpy()}
    ro, rl = oracle.decode_fp64(xc["q"], xc["k"].numpy(), xc["k_scale"].numpy(), xc["v"].numpy(),
                                xc["v_scale"].numpy(), xc["seq_lens"].numpy(), heads=heads, kv_format=fmt, **kw)
    og = o.double().cpu().numpy()
    lg = lse.double().cpu().numpy()
    sel = heads if heads is not None else [(b, h) for b in range(og.shape[0]) for h in range(og.shape[1])]
    bi = [b for b, _ in sel]
    hi = [h for _, h in sel]
    assert not np.isnan(og[bi, hi]).any()
    err_o = float(np.max(np.abs(og[bi, hi] - ro[bi, hi])))
    assert err_o <= TOL_O, f"O err {err_o}"
    assert np.array_equal(np.isneginf(lg[bi, hi]), np.isneginf(rl[bi, hi]))
    fin = np.isfinite(rl[bi, hi])
    err_l = float(np.max(np.abs(lg[bi, hi][fin] - rl[bi, hi][fin]), initial=0.0))
    assert err_l <= TOL_LSE, f"LSE err {err_l}"
    return err_o, err_l


def _make(B, Hq, Hkv, L, fmt, lens=None, W=0, rlens=None, seed=0):
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, 16, tuple(lens) if lens else (), fmt, W,
                                 tuple(rlens) if rlens else ())
    xc = fa_inputs.make_decode_inputs(cfg, seed=seed)
    return xc, {k: v.cuda() for k, v in xc.items()}


FP8_CASES = [
    # B, Hq, Hkv, L, lens, splits
    (1, 4, 1, 1, None, 1),
    (2, 8, 2, 100, [100, 37], 16),
    (3, 4, 4, 1000, [1000, 0, 513], 4),
    (2, 16, 1, 3000, [2999, 64], 16),
    (1, 32, 8, 4096, None, 16),
]


@pytest.mark.parametrize("B,Hq,Hkv,L,lens,splits", FP8_CASES)
def test_fp8_decode(gpu, B, Hq, Hkv, L, lens, splits):
    xc, x = _make(B, Hq, Hkv, L, "fp8", lens, seed=L + Hq + 1)
    o, lse = _decode(gpu, x, splits, False)
    print("max |dO|, |dLSE|", _compare(o, lse, xc, "fp8", False))


WINDOW_CASES = [
    # fmt, B, Hq, Hkv, L, lens, W, recent_lens, splits
    ("int8", 1, 4, 1, 64, None, 1, None, 2),
    ("int8", 2, 8, 2, 500, [500, 3], 37, [37, 5], 4),
    ("fp8", 3, 4, 1, 300, [300, 0, 0], 128, [0, 100, 0], 3),  # window only; nothing at all
    ("int8", 2, 16, 1, 1000, [999, 1000], 300, [300, 257], 16),
    ("fp8", 1, 32, 8, 2048, None, 128, None, 16),
]


@pytest.mark.parametrize("fmt,B,Hq,Hkv,L,lens,W,rlens,splits", WINDOW_CASES)
def test_window_decode(gpu, fmt, B, Hq, Hkv, L, lens, W, rlens, splits):
    xc, x = _make(B, Hq, Hkv, L, fmt, lens, W, rlens, seed=W + L)
    o, lse = _decode(gpu, x, splits, True)
    print("max |dO|, |dLSE|", _compare(o, lse, xc, fmt, True))


def test_window_without_lengths_attends_all(gpu):
    xc, x = _make(2, 4, 1, 200, "int8", None, 50, None, seed=11)
    B, Hq, d = x["q"].shape
    o = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    print("fa_decode_kvq window without recent_lens", flush=True)
    gpu.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse, seq_lens=x["seq_lens"],
                      num_splits=4, k_recent=x["k_recent"], v_recent=x["v_recent"])
    torch.cuda.synchronize()
    _compare(o, lse, xc, "int8", True)


@pytest.mark.parametrize("name", ["decode_fp8_b64_gqa32x8_L32768", "decode_int8_window128_b64_gqa32x8_L32768"])
def test_kv_decode_full_size(gpu, name):
    """The fp8-cache and window decode workloads at full size (B=64, 32/8 heads,
    L=32768, 16 splits), inputs drawn on the GPU, in the launch the benchmark
    times: every (batch, head) row of O and LSE against the oracle, and all of
    O checked for unwritten (NaN) elements."""
    cfg = fa_inputs.KV_CONFIGS[name]
    x = fa_inputs.make_decode_inputs(cfg, seed=0, device="cuda")
    window = cfg.W > 0
    o, lse = _decode(gpu, x, cfg.num_splits, window)
    assert not bool(torch.isnan(o.float()).any()) and not bool(torch.isnan(lse).any())
    xc = {k: v.cpu() for k, v in x.items()}
    del x
    torch.cuda.empty_cache()
    print(f"oracle decode, every row of {name}", flush=True)
    _compare(o, lse, xc, cfg.kv_format, window)


# ---- append, then decode ------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_append_then_decode(gpu, fmt):
    """Prefill rows appended into an empty cache in two chunks, the last rows kept
    as a bf16 window, then one decode step: equals the oracle's quantiser and
    decode applied to the same rows."""
    B, Hq, Hkv, L, d, W = 2, 8, 2, 256, 128, 16
    g = torch.Generator().manual_seed(21)
    krows = torch.randn(B, Hkv, 200, d, generator=g).to(torch.bfloat16)
    vrows = torch.randn(B, Hkv, 200, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    cdt = torch.int8 if fmt == "int8" else torch.uint8
    kc = torch.zeros(B, Hkv, L, d, dtype=cdt, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros(B, Hkv, L, dtype=torch.float16, device="cuda")
    vs = torch.zeros_like(ks)
    kr, vr = krows.cuda(), vrows.cuda()
    print(f"append then decode fmt={fmt}", flush=True)
    # chunk 1: rows 0..119, chunk 2: rows 120..183, window: rows 184..199
    gpu.fa_kv_append(kr[:, :, :120], vr[:, :, :120], kc, vc, ks, vs,
                     positions=torch.zeros(B, dtype=torch.int32, device="cuda"))
    gpu.fa_kv_append(kr[:, :, 120:184], vr[:, :, 120:184], kc, vc, ks, vs,
                     positions=torch.full((B,), 120, dtype=torch.int32, device="cuda"))
    lens = torch.full((B,), 184, dtype=torch.int32, device="cuda")
    o = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    gpu.fa_decode_kvq(q.cuda(), kc, vc, ks, vs, o, lse, seq_lens=lens, num_splits=4,
                      k_recent=kr[:, :, 184:].contiguous(), v_recent=vr[:, :, 184:].contiguous())
    torch.cuda.synchronize()
    qk, sk = oracle.quantize_kv_tokhead(krows[:, :, :184], fmt)
    qv, sv = oracle.quantize_kv_tokhead(vrows[:, :, :184], fmt)
    assert np.array_equal(kc[:, :, :184].cpu().numpy().view(np.uint8), qk.view(np.uint8))
    assert np.array_equal(vs[:, :, :184].cpu().numpy().view(np.uint16), sv.view(np.uint16))
    ro, rl = oracle.decode_fp64(q, qk, sk, qv, sv, None, kv_format=fmt,
                                k_recent=krows[:, :, 184:], v_recent=vrows[:, :, 184:])
    assert float(np.max(np.abs(o.double().cpu().numpy() - ro))) <= TOL_O
    assert float(np.max(np.abs(lse.double().cpu().numpy() - rl))) <= TOL_LSE
