"""Pins of the oracle's KV-cache write side and of its fp8-KV / residual-window
decode, against facts fixed outside the oracle: the E4M3FN value set (by
exhaustive search and by torch's float8_e4m3fn cast), the rounding bounds of
each format, closed forms, brute force on tiny inputs, and planted mistakes.
CPU only."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.e4m3 import e4m3_value
from oracle.quant import E4M3_QMAX, INT8_QMAX

FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)
FINITE_VALUES = np.array([e4m3_value(int(c)) for c in FINITE_CODES])


def _nearest_code_brute(x: float) -> int:
    """Nearest finite E4M3FN code by exhaustive search; a tie goes to the code
    whose mantissa is even; zero keeps the sign of x; beyond 448 saturates."""
    if abs(x) >= E4M3_QMAX:
        return 0x7E | (0x80 if x < 0 else 0)
    dist = np.abs(FINITE_VALUES - x)
    best = dist.min()
    cand = FINITE_CODES[dist == best]
    if len(cand) > 1:
        cand = np.array([c for c in cand if c & 1 == 0])
    vals = {e4m3_value(int(c)) for c in cand}
    if vals == {0.0}:  # +0 and -0: keep the sign of x
        return 0x80 if math.copysign(1.0, x) < 0 else 0x00
    # otherwise the candidates share one value and the sign of x
    for c in cand:
        if (c >> 7) == (1 if x < 0 else 0):
            return int(c)
    return int(cand[0])


# ---- E4M3FN encoder -----------------------------------------------------------

def test_e4m3_encode_round_trips_every_finite_code():
    enc = oracle.e4m3_encode(FINITE_VALUES)
    assert np.array_equal(enc.astype(np.int64), FINITE_CODES)


def test_e4m3_encode_matches_exhaustive_nearest_search():
    rng = np.random.default_rng(7)
    # values in every binade, exact midpoints between neighbours, tiny values
    xs = list(rng.standard_normal(400) * 40) + list(rng.standard_normal(200) * 0.02)
    fv = np.sort(np.unique(FINITE_VALUES))
    xs += list((fv[1:] + fv[:-1]) / 2)  # every tie point
    xs += [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 447.9, -447.9, 448.0, 1e-30]
    enc = oracle.e4m3_encode(np.array(xs))
    for x, c in zip(xs, enc):
        assert int(c) == _nearest_code_brute(x), (x, int(c))


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(5000) * 1e-2])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(ref, ours)


# ---- per-token-per-head quantisers --------------------------------------------

def _rows(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_quantiser_error_bound_and_absmax(fmt):
    x = _rows((2, 3, 50, 128), 11)
    x[0, 0, 3] = 0  # an all-zero row
    x[1, 2, 7] *= 1e4  # a large row
    codes, sc = oracle.quantize_kv_tokhead(x, fmt)
    xf = x.float().numpy().astype(np.float64)
    scf = sc.astype(np.float64)
    deq = (codes.astype(np.float64) if fmt == "int8" else oracle.e4m3_decode(codes)) * scf[..., None]
    amax = np.abs(xf).max(axis=-1)
    qmax = INT8_QMAX if fmt == "int8" else E4M3_QMAX
    # the scale is a nearest fp16 to absmax / QMAX (up to the fp32 step before it)
    rel = np.abs(scf - amax / qmax) / np.maximum(amax / qmax, 1e-300)
    assert np.all(rel[amax > 0] <= 2.0 ** -11 * (1 + 2.0 ** -12))
    assert np.all(sc[0, 0, 3] == 0) and np.all(codes[0, 0, 3] == 0)
    if fmt == "int8":
        assert np.all(np.abs(codes.astype(np.int64)) <= 127)
        # half a code step, plus the fp32 rounding of x / sc
        assert np.all(np.abs(xf - deq) <= scf[..., None] * (0.5 + 1e-5))
    else:
        y = np.abs(xf) / np.where(scf > 0, scf, 1)[..., None]
        # half the spacing of the binade of y (2^-9 below 2^-6), relative slack for fp32
        e = np.clip(np.floor(np.log2(np.where(y > 0, y, 1))), -6, 8)
        half = np.exp2(e - 4)
        assert np.all(np.abs(xf - deq) <= (half + y * 2e-7) * scf[..., None] + 1e-300)
    # the absmax element of every live row maps to +-QMAX exactly
    live = scf > 0
    idx = np.abs(xf).argmax(axis=-1)
    top = np.take_along_axis(codes, idx[..., None], axis=-1)[..., 0]
    if fmt == "int8":
        assert np.all(np.abs(top[live].astype(np.int64)) == 127)
    else:
        assert np.all((top[live] & 0x7F) == 0x7E)


def test_int8_quantiser_matches_exhaustive_search():
    x = _rows((1, 2, 9, 16), 12)
    codes, sc = oracle.quantize_kv_tokhead(x, "int8")
    xf = x.float().numpy()
    cand = np.arange(-127, 128)
    for h in range(2):
        for t in range(9):
            s = np.float32(sc[0, h, t])
            for c in range(16):
                y = float(np.float32(xf[0, h, t, c]) / s)  # the fp32 division of the reading
                dist = np.abs(cand - y)
                best = cand[dist == dist.min()]
                want = best[best % 2 == 0][0] if len(best) > 1 else best[0]
                assert codes[0, h, t, c] == want


def test_fp8_quantiser_matches_torch_on_the_same_quotient():
    x = _rows((2, 2, 40, 128), 13, scale=3.0)
    codes, sc = oracle.quantize_kv_tokhead(x, "fp8")
    xf = x.float()
    s = torch.from_numpy(sc.astype(np.float32))
    y = (xf / s[..., None]).clamp(-448, 448)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, codes)


def test_scale_saturates_and_underflows():
    x = torch.zeros(1, 1, 3, 128, dtype=torch.float32)
    x[0, 0, 0, 5] = 3e38  # absmax / 127 beyond fp16: scale saturates at 65504
    x[0, 0, 1, 9] = 1e-12  # scale underflows fp16 to zero: codes are zero
    x[0, 0, 2, 0] = -1.0
    for fmt in ("int8", "fp8"):
        codes, sc = oracle.quantize_kv_tokhead(x.numpy(), fmt)
        assert float(sc[0, 0, 0]) == 65504.0
        assert float(sc[0, 0, 1]) == 0.0 and np.all(codes[0, 0, 1] == 0)
        top = codes[0, 0, 0, 5]
        assert (int(top) == 127) if fmt == "int8" else (int(top) == 0x7E)
        neg = codes[0, 0, 2, 0]
        assert (int(neg) == -127) if fmt == "int8" else (int(neg) == 0xFE)


def test_append_places_rows_and_drops_out_of_range_slots():
    B, H, L, T, d = 3, 2, 10, 4, 8
    x = _rows((B, H, T, d), 14)
    codes0 = np.full((B, H, L, d), 0x55, dtype=np.uint8)
    sc0 = np.full((B, H, L), 7.0, dtype=np.float16)
    pos = np.array([0, 8, -2])
    codes, sc = oracle.kv_append_ref(codes0, sc0, x, pos, "fp8")
    qc, qs = oracle.quantize_kv_tokhead(x, "fp8")
    assert np.array_equal(codes[0, :, 0:4], qc[0]) and np.array_equal(sc[0, :, 0:4], qs[0])
    assert np.all(codes[0, :, 4:] == 0x55) and np.all(sc[0, :, 4:] == 7.0)
    assert np.array_equal(codes[1, :, 8:10], qc[1, :, 0:2]) and np.all(codes[1, :, :8] == 0x55)
    assert np.array_equal(codes[2, :, 0:2], qc[2, :, 2:4]) and np.all(codes[2, :, 2:] == 0x55)


# ---- fp8-KV and residual-window decode ------------------------------------------

def test_fp8_decode_equals_brute_force_on_decoded_values():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, L, d = 2, 4, 2, 11, 8
    kc = rng.choice(FINITE_CODES, (B, Hkv, L, d)).astype(np.uint8)
    vc = rng.choice(FINITE_CODES, (B, Hkv, L, d)).astype(np.uint8)
    ks = (rng.random((B, Hkv, L)) * 0.01).astype(np.float16)
    vs = (rng.random((B, Hkv, L)) * 0.01).astype(np.float16)
    q = rng.standard_normal((B, Hq, d))
    lens = [11, 5]
    o, lse = oracle.decode_fp64(q, kc, ks, vc, vs, lens, kv_format="fp8")
    for b in range(B):
        n = lens[b]
        kb = [[[[e4m3_value(int(kc[b, hh, t, c])) * float(ks[b, hh, t]) for c in range(d)] for t in range(n)]
               for hh in range(Hkv)]]
        vb = [[[[e4m3_value(int(vc[b, hh, t, c])) * float(vs[b, hh, t]) for c in range(d)] for t in range(n)]
               for hh in range(Hkv)]]
        ob, lb = oracle.attention_brute([[[list(q[b, h])] for h in range(Hq)]], kb, vb, False)
        for h in range(Hq):
            assert np.max(np.abs(np.array(ob[0][h][0]) - o[b, h])) < 1e-12
            assert abs(lb[0][h][0] - lse[b, h]) < 1e-12


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_window_equals_brute_force_over_cache_and_window(fmt):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, L, W, d = 2, 4, 1, 9, 5, 8
    x = _rows((B, Hkv, L, d), 23)
    kc, ks = oracle.quantize_kv_tokhead(x, fmt)
    vc, vs = oracle.quantize_kv_tokhead(_rows((B, Hkv, L, d), 24), fmt)
    kr = _rows((B, Hkv, W, d), 25)
    vr = _rows((B, Hkv, W, d), 26)
    q = rng.standard_normal((B, Hq, d))
    lens, rl = [9, 0], [3, 5]
    o, lse = oracle.decode_fp64(q, kc, ks, vc, vs, lens, kv_format=fmt, k_recent=kr, v_recent=vr, recent_lens=rl)
    deq = oracle.dequant_int8_fp64 if fmt == "int8" else oracle.dequant_fp8_fp64
    for b in range(B):
        kk = np.concatenate([deq(kc[b, 0, :lens[b]], ks[b, 0, :lens[b]]), kr[b, 0, :rl[b]].double().numpy()])
        vv = np.concatenate([deq(vc[b, 0, :lens[b]], vs[b, 0, :lens[b]]), vr[b, 0, :rl[b]].double().numpy()])
        ob, lb = oracle.attention_brute([[[list(q[b, h])] for h in range(Hq)]], [[kk.tolist()]], [[vv.tolist()]], False)
        for h in range(Hq):
            assert np.max(np.abs(np.array(ob[0][h][0]) - o[b, h])) < 1e-12
            assert abs(lb[0][h][0] - lse[b, h]) < 1e-12


def test_window_zero_query_closed_form():
    # q = 0: every visible key has the same score, so O is the mean of all
    # visible values (cache and window together) and LSE = ln(count)
    B, Hkv, L, W, d = 1, 1, 6, 4, 8
    kc, ks = oracle.quantize_kv_tokhead(_rows((B, Hkv, L, d), 27), "int8")
    vc, vs = oracle.quantize_kv_tokhead(_rows((B, Hkv, L, d), 28), "int8")
    kr, vr = _rows((B, Hkv, W, d), 29), _rows((B, Hkv, W, d), 30)
    q = np.zeros((B, 2, d))
    o, lse = oracle.decode_fp64(q, kc, ks, vc, vs, [4], k_recent=kr, v_recent=vr, recent_lens=[3])
    vals = np.concatenate([vc[0, 0, :4].astype(np.float64) * vs[0, 0, :4, None].astype(np.float64),
                           vr[0, 0, :3].double().numpy()])
    assert np.max(np.abs(o[0, 0] - vals.mean(axis=0))) < 1e-12
    assert abs(lse[0, 1] - math.log(7)) < 1e-12


def test_token_moved_from_window_into_cache_changes_nothing():
    # a window row that is exactly representable as code x scale gives the same
    # result whether it sits in the window or in the cache
    B, Hkv, L, W, d = 1, 1, 5, 2, 8
    kc, ks = oracle.quantize_kv_tokhead(_rows((B, Hkv, L, d), 31), "int8")
    vc, vs = oracle.quantize_kv_tokhead(_rows((B, Hkv, L, d), 32), "int8")
    q = np.random.default_rng(33).standard_normal((B, 2, d))
    kr = torch.zeros(B, Hkv, W, d, dtype=torch.bfloat16)
    vr = torch.zeros(B, Hkv, W, d, dtype=torch.bfloat16)
    kr[0, 0, 0] = torch.from_numpy(kc[0, 0, 4].astype(np.float32) * np.float32(ks[0, 0, 4])).to(torch.bfloat16)
    vr[0, 0, 0] = torch.from_numpy(vc[0, 0, 4].astype(np.float32) * np.float32(vs[0, 0, 4])).to(torch.bfloat16)
    exact = (kr[0, 0, 0].double().numpy() == kc[0, 0, 4] * float(ks[0, 0, 4])).all() and \
        (vr[0, 0, 0].double().numpy() == vc[0, 0, 4] * float(vs[0, 0, 4])).all()
    if not exact:  # pick scales for which the products fit bf16 exactly
        ks[0, 0, 4] = vs[0, 0, 4] = np.float16(0.0078125)
        kr[0, 0, 0] = torch.from_numpy(kc[0, 0, 4].astype(np.float32) / 128).to(torch.bfloat16)
        vr[0, 0, 0] = torch.from_numpy(vc[0, 0, 4].astype(np.float32) / 128).to(torch.bfloat16)
    o1, l1 = oracle.decode_fp64(q, kc, ks, vc, vs, [5])
    o2, l2 = oracle.decode_fp64(q, kc, ks, vc, vs, [4], k_recent=kr, v_recent=vr, recent_lens=[1])
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


# ---- planted mistakes in the write side are caught ---------------------------------

def _mutant_quant(kind):
    def run(x, fmt):
        xf = x.float().numpy() if hasattr(x, "float") else np.asarray(x, np.float32)
        qmax = np.float32(127 if fmt == "int8" else 448)
        if kind == "qmax_128":
            qmax = np.float32(128 if fmt == "int8" else 480)
        amax = np.abs(xf).max(axis=-1)
        if kind == "amax_signed":
            amax = xf.max(axis=-1)
        sc = (amax / qmax).astype(np.float16)
        scf = np.where(sc > 0, sc.astype(np.float32), 1)
        y = xf / scf[..., None]
        if kind == "multiply_not_divide":
            y = xf * scf[..., None]
        if fmt == "int8":
            r = np.floor(y + 0.5) if kind == "round_half_up" else np.rint(y)
            if kind == "truncate":
                r = np.trunc(y)
            return np.clip(r, -127, 127).astype(np.int8), sc
        c = oracle.e4m3_encode(np.clip(y, -448, 448).astype(np.float64))
        if kind == "truncate":
            c = oracle.e4m3_encode(np.trunc(np.clip(y, -448, 448) * 8) / 8)
        return c, sc

    return run


@pytest.mark.parametrize("kind", ["qmax_128", "amax_signed", "multiply_not_divide", "round_half_up", "truncate"])
def test_planted_quantiser_mistakes_are_caught(kind):
    run = _mutant_quant(kind)
    caught = False
    for fmt in ("int8", "fp8"):
        x = _rows((1, 2, 64, 128), 40)
        # a row with exact ties: absmax 127/16 gives the scale 1/16 exactly, and
        # these entries divide to y = 0.5, 1.5, 2.5, -0.5
        x[0, 0, 0] = 0
        x[0, 0, 0, 4] = 127 / 16
        x[0, 0, 0, :4] = torch.tensor([0.5, 1.5, 2.5, -0.5]) / 16
        codes, sc = run(x, fmt)
        xf = x.float().numpy().astype(np.float64)
        scf = sc.astype(np.float64)
        deq = (codes.astype(np.float64) if fmt == "int8" else oracle.e4m3_decode(codes)) * scf[..., None]
        amax = np.abs(xf).max(axis=-1)
        qmax = 127 if fmt == "int8" else 448
        bad_scale = np.any(np.abs(scf - amax / qmax) > amax / qmax * 2.0 ** -10)
        if fmt == "int8":
            bad_err = np.any(np.abs(xf - deq) > scf[..., None] * (0.5 + 1e-5))
            # the brute-force search decides the codes exactly
            cand = np.arange(-127, 128)
            bad_brute = False
            for c in range(8):
                y = float(np.float32(xf[0, 0, 0, c]) / np.float32(sc[0, 0, 0]))
                d = np.abs(cand - y)
                best = cand[d == d.min()]
                want = best[best % 2 == 0][0] if len(best) > 1 else best[0]
                bad_brute |= codes[0, 0, 0, c] != want
        else:
            y = np.abs(xf) / np.where(scf > 0, scf, 1)[..., None]
            e = np.clip(np.floor(np.log2(np.where(y > 0, y, 1))), -6, 8)
            bad_err = np.any(np.abs(xf - deq) > (np.exp2(e - 4) + y * 2e-7) * scf[..., None])
            bad_brute = False
        caught |= bool(bad_scale or bad_err or bad_brute)
    assert caught, f"mutant {kind} slipped through"


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float16])
def test_code_boundaries_are_hit_exactly_or_missed_by_a_margin(fmt, in_dtype):
    """The margin the append kernel's quotient relies on: for bf16/fp16 x and
    an fp16 scale sc, x - t * sc (t the code's rounding boundary nearest x / sc:
    an int8 half-integer, an E4M3 midpoint, or the clamp) is either exactly 0
    or at least 2^-20 |x|, so a quotient within a few fp32 ulps (2^-23) of
    x / sc that is exact on the boundary decides every code as the correctly
    rounded quotient does.  Checked on the boundary rows of the GPU test, in
    float64, where t * sc (at most 20 significant bits) and the difference are
    exact."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from kv_boundary import boundary_rows

    rows = boundary_rows(fmt, in_dtype, 1024, seed=31)
    _, sc = oracle.quantize_kv_tokhead(rows, fmt)
    x = rows.double().numpy()
    s = sc.astype(np.float64)[:, None]
    qmax = INT8_QMAX if fmt == "int8" else E4M3_QMAX
    if fmt == "int8":
        bnd = np.arange(128) + 0.5
    else:
        vals = np.unique([abs(e4m3_value(c)) for c in range(256) if math.isfinite(e4m3_value(c))])
        bnd = (vals[1:] + vals[:-1]) / 2
    bnd = np.concatenate([bnd[bnd < qmax], [qmax]])
    ay = np.abs(x) / s
    i = np.clip(np.searchsorted(bnd, ay), 1, len(bnd) - 1)
    dist = np.minimum(np.abs(np.abs(x) - bnd[i] * s), np.abs(np.abs(x) - bnd[i - 1] * s))
    nz = (dist > 0) & (x != 0)
    assert int((dist == 0).sum()) > 1000                      # plenty of exact ties in the rows
    assert np.all(dist[nz] >= 2.0 ** -20 * np.abs(x[nz]))
