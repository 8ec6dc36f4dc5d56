"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check is independent of the oracle's own code path: brute force with
correctly rounded scalar sums, closed forms, invariants, a library routine on a
special case, and a hand-derived instance of the pages' two-tile exercise.  A
final test plants plausible mistakes in copies of the oracle and checks that
these pins catch every one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import _two_pass_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


TINY = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 1, 1, 1, 1, 1, False),
    (1, 1, 1, 5, 7, 3, False),
    (2, 2, 1, 4, 4, 4, True),
    (1, 4, 2, 9, 9, 8, True),
    (2, 2, 2, 6, 11, 5, True),   # Sq < Sk: bottom-right causal
    (1, 2, 1, 7, 3, 2, True),    # Sq > Sk: leading rows see no key
    (1, 3, 3, 17, 17, 8, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,causal", TINY)
def test_numpy_matches_brute_force(B, Hq, Hkv, Sq, Sk, d, causal):
    q = rnd((B, Hq, Sq, d), 1)
    k = rnd((B, Hkv, Sk, d), 2)
    v = rnd((B, Hkv, Sk, d + 1), 3)
    o, lse = oracle.attention_fp64(q, k, v, causal)
    ob, lb = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), causal)
    ob = np.array(ob)
    lb = np.array(lb)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-12


def test_library_special_case_sdpa():
    """Equal heads, no mask offsets: torch's float64 CPU SDPA and logsumexp."""
    q = torch.randn(2, 3, 33, 16, dtype=torch.float64)
    k = torch.randn(2, 3, 40, 16, dtype=torch.float64)
    v = torch.randn(2, 3, 40, 16, dtype=torch.float64)
    o, lse = oracle.attention_fp64(q, k, v, False)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    ref_lse = torch.logsumexp(q @ k.transpose(-1, -2) / 4.0, dim=-1)
    assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-12
    # causal with Sq == Sk is the library's lower-triangular mask
    q2 = q[:, :, :20]
    k2, v2 = k[:, :, :20], v[:, :, :20]
    o2, _ = oracle.attention_fp64(q2, k2, v2, True)
    ref2 = torch.nn.functional.scaled_dot_product_attention(q2, k2, v2, is_causal=True)
    assert np.max(np.abs(o2 - ref2.numpy())) < 1e-12


def test_zero_query_gives_mean_of_visible_values():
    B, H, S, d = 1, 2, 12, 4
    q = np.zeros((B, H, S, d))
    k = rnd((B, H, S, d), 5)
    v = rnd((B, H, S, d), 6)
    o, lse = oracle.attention_fp64(q, k, v, True)
    for i in range(S):
        assert np.allclose(o[0, :, i], v[0, :, : i + 1].mean(axis=1), atol=1e-13)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-13
    o, lse = oracle.attention_fp64(q, k, v, False)
    assert np.allclose(o[0, :, 3], v[0].mean(axis=1), atol=1e-13)
    assert np.allclose(lse, math.log(S), atol=1e-13)


def test_single_key_returns_its_value_row():
    q = rnd((1, 2, 5, 8), 7)
    k = rnd((1, 2, 1, 8), 8)
    v = rnd((1, 2, 1, 8), 9)
    o, lse = oracle.attention_fp64(q, k, v, False)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    s00 = np.einsum("bhid,bhjd->bhij", q, k)[..., 0] / math.sqrt(8)
    assert np.allclose(lse, s00, atol=1e-13)


def test_constant_value_rows_return_that_row():
    q = rnd((2, 2, 9, 8), 10)
    k = rnd((2, 2, 13, 8), 11)
    row = rnd((8,), 12)
    v = np.broadcast_to(row, (2, 2, 13, 8)).copy()
    for causal in (False, True):
        o, _ = oracle.attention_fp64(q, k, v, causal)
        assert np.allclose(o, np.broadcast_to(row, o.shape), atol=1e-13)


def test_dominant_key_selects_its_value_row():
    d = 8
    q = rnd((1, 1, 4, d), 13)
    k = rnd((1, 1, 10, d), 14) * 0.1
    v = rnd((1, 1, 10, d), 15)
    jstar = 6
    k[0, 0, jstar] = q[0, 0, 2] * 400.0  # score gap far above 50 for row 2
    o, _ = oracle.attention_fp64(q, k, v, False)
    assert np.max(np.abs(o[0, 0, 2] - v[0, 0, jstar])) < 1e-18 + math.exp(-50) * 10


def test_causal_first_row_is_first_value():
    q = rnd((1, 2, 6, 4), 16)
    k = rnd((1, 2, 6, 4), 17)
    v = rnd((1, 2, 6, 4), 18)
    o, _ = oracle.attention_fp64(q, k, v, True)
    assert np.array_equal(o[0, :, 0], v[0, :, 0])


def test_empty_rows_zero_output_minus_inf_lse():
    q = rnd((1, 1, 6, 4), 19)
    k = rnd((1, 1, 3, 4), 20)
    v = rnd((1, 1, 3, 4), 21)
    o, lse = oracle.attention_fp64(q, k, v, True)  # rows 0..2 see nothing
    assert np.all(o[0, 0, :3] == 0) and np.all(np.isneginf(lse[0, 0, :3]))
    assert np.all(np.isfinite(lse[0, 0, 3:]))


def test_probability_rows_sum_to_one_and_lse_bounds():
    q = rnd((1, 2, 10, 6), 22, 3.0)
    k = rnd((1, 1, 10, 6), 23, 3.0)
    v = rnd((1, 1, 10, 6), 24)
    for causal in (False, True):
        p = oracle.attention_probs_fp64(q, k, causal)
        assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-12)
        o, lse = oracle.attention_fp64(q, k, v, causal)
        assert np.allclose(o, p @ v[:, [0, 0]], atol=1e-12)
        s = np.einsum("bhid,bjd->bhij", q, k[:, 0]) / math.sqrt(6)
        for i in range(10):
            n = oracle.visible_keys(i, 10, 10, causal)
            m = s[..., i, :n].max(axis=-1)
            assert np.all(m <= lse[..., i] + 1e-12)
            assert np.all(lse[..., i] <= m + math.log(n) + 1e-12)


@pytest.mark.parametrize("bk", [1, 3, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_two_pass(bk, causal):
    q = rnd((1, 2, 70, 8), 25, 2.0)
    k = rnd((1, 2, 70, 8), 26, 2.0)
    v = rnd((1, 2, 70, 8), 27)
    o, lse = oracle.attention_fp64(q, k, v, causal)
    o2, lse2 = oracle.online_softmax_fp64(q, k, v, causal, block_q=16, block_k=bk)
    assert np.max(np.abs(o - o2)) < 1e-12
    assert np.max(np.abs(lse - lse2)) < 1e-12


def test_online_recurrence_with_empty_rows():
    q = rnd((1, 1, 9, 4), 28)
    k = rnd((1, 1, 5, 4), 29)
    v = rnd((1, 1, 5, 4), 30)
    o, lse = oracle.attention_fp64(q, k, v, True)
    o2, lse2 = oracle.online_softmax_fp64(q, k, v, True, block_q=4, block_k=2)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse2))
    assert np.max(np.abs(o - o2)) < 1e-12


def test_two_tile_exercise_golden():
    g = json.load(open(os.path.join(HERE, "golden", "two_tile_exercise.json")))
    a, b = g["a"], g["b"]
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    k = np.array([[[[math.log(x), math.log(y)] for x, y in zip(a, b)]]])
    v = np.array([[g["v"]]], dtype=np.float64)
    trace = []
    o, lse = oracle.online_softmax_fp64(q, k, v, False, scale=1.0, block_q=2, block_k=2, trace=trace)
    assert len(trace) == 2
    for (m, l, acc), key in zip(trace, ["tile1", "tile2"]):
        assert np.allclose(np.exp(m), g[key]["m_exp"], atol=1e-12)
        assert np.allclose(l, g[key]["l"], atol=1e-12)
        assert np.allclose(acc, g[key]["o_unnorm"], atol=1e-12)
    assert np.allclose(o[0, 0], g["final"]["o"], atol=1e-12)
    assert np.allclose(np.exp(lse[0, 0]), g["final"]["lse_exp"], atol=1e-11)
    o2, lse2 = oracle.attention_fp64(q, k, v, False, scale=1.0)
    assert np.allclose(o2[0, 0], g["final"]["o"], atol=1e-12)


def test_row_selection_matches_full_evaluation():
    q = rnd((1, 4, 40, 8), 60)
    k = rnd((1, 2, 40, 8), 61)
    v = rnd((1, 2, 40, 8), 62)
    rows = [0, 5, 17, 39]
    for causal in (False, True):
        o, lse = oracle.attention_fp64(q, k, v, causal)
        o2, lse2 = oracle.attention_fp64(q, k, v, causal, rows=rows, heads=[(0, 1), (0, 3)])
        for h in (1, 3):
            assert np.array_equal(o2[0, h], o[0, h, rows]) and np.array_equal(lse2[0, h], lse[0, h, rows])
        assert np.all(o2[0, 0] == 0) and np.all(np.isneginf(lse2[0, 2]))


def test_key_value_permutation_invariance():
    q = rnd((1, 2, 8, 6), 31)
    k = rnd((1, 2, 15, 6), 32)
    v = rnd((1, 2, 15, 6), 33)
    perm = np.random.default_rng(34).permutation(15)
    o, lse = oracle.attention_fp64(q, k, v, False)
    o2, lse2 = oracle.attention_fp64(q, k[:, :, perm], v[:, :, perm], False)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


def test_gqa_equals_mha_with_repeated_kv_heads():
    q = rnd((2, 8, 7, 4), 35)
    k = rnd((2, 2, 9, 4), 36)
    v = rnd((2, 2, 9, 4), 37)
    o, lse = oracle.attention_fp64(q, k, v, True)
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    o2, lse2 = oracle.attention_fp64(q, kr, vr, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # and the head mapping is h // G (heads 0..3 share kv head 0)
    o3, _ = oracle.attention_fp64(q[:, :4], k[:, :1], v[:, :1], True)
    assert np.array_equal(o[:, :4], o3)


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_split_and_merge_equals_unsplit(splits):
    q = rnd((2, 2, 3, 8), 38, 2.0)
    k = rnd((2, 2, 37, 8), 39, 2.0)
    v = rnd((2, 2, 37, 8), 40)
    o, lse = oracle.attention_fp64(q, k, v, False)
    o2, lse2 = oracle.split_merge_fp64(q, k, v, splits)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12
    if splits == 1:
        assert np.array_equal(o, o2)


def test_split_with_empty_chunks():
    q = rnd((1, 1, 2, 4), 41)
    k = rnd((1, 1, 5, 4), 42)
    v = rnd((1, 1, 5, 4), 43)
    o, lse = oracle.attention_fp64(q, k, v, False)
    o2, lse2 = oracle.split_merge_fp64(q, k, v, 4)  # chunk 2: keys 0-1,2-3,4,(empty)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


def test_decode_oracle_dequantises_then_attends():
    rng = np.random.default_rng(44)
    B, Hq, Hkv, L, d = 2, 4, 2, 19, 8
    kc = rng.integers(-127, 128, (B, Hkv, L, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, L, d)).astype(np.int8)
    ks = (rng.random((B, Hkv, L)) * 0.05).astype(np.float16)
    vs = (rng.random((B, Hkv, L)) * 0.05).astype(np.float16)
    q = rnd((B, Hq, d), 45)
    lens = [19, 7]
    o, lse = oracle.decode_fp64(q, kc, ks, vc, vs, lens)
    # brute force per (b, h) over the dequantised prefix
    for b in range(B):
        n = lens[b]
        kf = [[float(kc[b, hh, t, c]) * float(ks[b, hh, t]) for c in range(d)] for hh in range(Hkv) for t in range(n)]
        vf = [[float(vc[b, hh, t, c]) * float(vs[b, hh, t]) for c in range(d)] for hh in range(Hkv) for t in range(n)]
        kb = [[kf[hh * n:(hh + 1) * n] for hh in range(Hkv)]]
        vb = [[vf[hh * n:(hh + 1) * n] for hh in range(Hkv)]]
        ob, lb = oracle.attention_brute([[[list(q[b, h])] for h in range(Hq)]], kb, vb, False)
        for h in range(Hq):
            assert np.max(np.abs(np.array(ob[0][h][0]) - o[b, h])) < 1e-12
            assert abs(lb[0][h][0] - lse[b, h]) < 1e-12
    # a zero-length sequence gives O = 0, LSE = -inf
    o0, l0 = oracle.decode_fp64(q, kc, ks, vc, vs, [0, 3])
    assert np.all(o0[0] == 0) and np.all(np.isneginf(l0[0]))


def test_dequant_is_exact_product():
    codes = np.array([[-127, 0, 5, 127]], dtype=np.int8)
    sc = np.array([np.float16(0.0234)], dtype=np.float16)
    out = oracle.dequant_int8_fp64(codes, sc)
    assert np.array_equal(out[0], codes[0].astype(np.float64) * float(sc[0]))


# ---- e4m3 decoder pins ------------------------------------------------------

def test_e4m3_decoder_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.sum(nan) == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], ours[~nan])


def test_e4m3_decoder_closed_forms():
    from oracle.e4m3 import e4m3_value

    assert e4m3_value(0x7E) == 448.0 and e4m3_value(0xFE) == -448.0
    assert e4m3_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert e4m3_value(0x08) == 2.0 ** -6  # smallest normal
    assert e4m3_value(0x38) == 1.0
    assert e4m3_value(0x80) == 0.0 and math.copysign(1, e4m3_value(0x80)) == -1


# ---- the pins must catch planted mistakes ------------------------------------

def _mutant(kind):
    """A copy of the two-pass oracle with one plausible mistake planted."""

    def run(q, k, v, causal, scale=None):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        tau = 1.0 / math.sqrt(d)
        if kind == "no_scale":
            tau = 1.0
        if kind == "scale_1_over_d":
            tau = 1.0 / d
        o = np.zeros((B, Hq, Sq, v.shape[3]))
        lse = np.full((B, Hq, Sq), -np.inf)
        for b in range(B):
            for h in range(Hq):
                kvh = h % Hkv if kind == "gqa_mod" else h // G
                kk, vv = k[b, kvh], v[b, kvh]
                if kind == "swap_kv":
                    kk, vv = vv, kk
                n_vis = np.array([oracle.visible_keys(i, Sq, Sk, causal) for i in range(Sq)])
                if kind == "causal_top_left":
                    n_vis = np.array([min(Sk, i + 1) if causal else Sk for i in range(Sq)])
                if kind == "causal_strict":
                    n_vis = np.maximum(n_vis - (1 if causal else 0), 0)
                qq = q[b, h]
                if kind == "transpose_q":
                    qq = qq[::-1]
                oo, ll = _two_pass_rows(qq, kk, vv, tau, n_vis, 4)
                if kind == "lse_no_max":
                    ll = ll - np.where(np.isfinite(ll), (qq @ kk.T * tau).max(axis=1), 0)
                if kind == "lse_log2":
                    ll = ll / math.log(2)
                if kind == "no_normalise":  # forgets the final division by l
                    s = (qq @ kk.T) * tau
                    vis = np.arange(Sk)[None, :] < n_vis[:, None]
                    s = np.where(vis, s, -np.inf)
                    m = np.where(n_vis > 0, s.max(axis=1), 0.0)
                    oo = np.where(vis, np.exp(s - m[:, None]), 0.0) @ vv
                o[b, h], lse[b, h] = oo, ll
        return o, lse

    return run


MUTANTS = ["no_scale", "scale_1_over_d", "gqa_mod", "swap_kv", "causal_top_left",
           "causal_strict", "transpose_q", "lse_no_max", "lse_log2", "no_normalise"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind):
    run = _mutant(kind)
    caught = []
    # brute force on shapes that exercise every axis
    for (B, Hq, Hkv, Sq, Sk, d, causal) in [(1, 4, 2, 5, 8, 4, True), (1, 2, 1, 4, 4, 3, False)]:
        q = rnd((B, Hq, Sq, d), 50)
        k = rnd((B, Hkv, Sk, d), 51)
        v = rnd((B, Hkv, Sk, d), 52)
        o, lse = run(q, k, v, causal)
        ob, lb = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), causal)
        ob, lb = np.array(ob), np.array(lb)
        fin = np.isfinite(lb)
        bad = (not np.array_equal(np.isfinite(lse), fin)) or np.max(np.abs(o - ob)) > 1e-9 \
            or np.max(np.abs(lse[fin] - lb[fin])) > 1e-9
        caught.append(bad)
    # closed form: zero query -> running mean, LSE = ln(i+1)
    q = np.zeros((1, 1, 6, 4))
    k = rnd((1, 1, 6, 4), 53)
    v = rnd((1, 1, 6, 4), 54)
    o, lse = run(q, k, v, True)
    want = np.array([v[0, 0, : i + 1].mean(axis=0) for i in range(6)])
    caught.append(np.max(np.abs(o[0, 0] - want)) > 1e-9
                  or np.max(np.abs(lse[0, 0] - np.log(np.arange(1, 7)))) > 1e-9)
    assert any(caught), f"mutant {kind} slipped through every pin"
