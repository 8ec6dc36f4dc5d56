"""Pins of the oracle's attention backward against facts fixed outside it:
central finite differences of the (separately pinned) forward oracle, torch's
float64 autograd through a plain softmax attention, closed forms, invariants
that follow from the softmax, and planted mistakes.  CPU only."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import visible_keys


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


SHAPES = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 1, 1, 4, 4, 3, False),
    (1, 2, 1, 5, 7, 4, True),
    (2, 4, 2, 6, 6, 3, True),
    (1, 2, 2, 7, 3, 2, True),   # Sq > Sk: leading rows see no key
]


def _loss(q, k, v, do, causal):
    o, _ = oracle.attention_fp64(q, k, v, causal, threads=1)
    return float(np.sum(o * do))


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,causal", SHAPES)
def test_backward_matches_central_differences(B, Hq, Hkv, Sq, Sk, d, causal):
    q, k, v = rnd((B, Hq, Sq, d), 1), rnd((B, Hkv, Sk, d), 2), rnd((B, Hkv, Sk, d), 3)
    do = rnd((B, Hq, Sq, d), 4)
    dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(q, k, v, do, causal)
            x[idx] = keep - h
            lm = _loss(q, k, v, do, causal)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(g)))


def test_backward_matches_torch_autograd():
    B, Hq, Hkv, Sq, Sk, d = 2, 4, 2, 9, 11, 8
    for causal in (False, True):
        q, k, v = rnd((B, Hq, Sq, d), 5), rnd((B, Hkv, Sk, d), 6), rnd((B, Hkv, Sk, d), 7)
        do = rnd((B, Hq, Sq, d), 8)
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        G = Hq // Hkv
        kk = tk.repeat_interleave(G, dim=1)
        vv = tv.repeat_interleave(G, dim=1)
        s = (tq @ kk.transpose(-1, -2)) / math.sqrt(d)
        if causal:  # bottom-right aligned mask, as the forward reads it
            mask = torch.tensor([[j >= visible_keys(i, Sq, Sk, True) for j in range(Sk)] for i in range(Sq)])
            s = s.masked_fill(mask, float("-inf"))
        o = torch.softmax(s, dim=-1) @ vv
        o.backward(torch.tensor(do))
        dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, causal)
        for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(ours - ref.numpy())) < 1e-12


def test_constant_values_give_zero_query_and_key_gradients():
    # every value row equal: O does not depend on P, so dQ = dK = 0 and
    # dV_j = sum_i P_ij dO_i sums (over j) to sum_i dO_i
    B, Hq, S, d = 1, 2, 6, 4
    q, k = rnd((B, Hq, S, d), 9), rnd((B, Hq, S, d), 10)
    v = np.tile(rnd((1, 1, 1, d), 11), (B, Hq, S, 1))
    do = rnd((B, Hq, S, d), 12)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, causal)
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) < 1e-12


def test_single_key_closed_form():
    # one key: P = 1 for every row, so dQ = dK = 0 and dV_0 = sum_i dO_i
    q, k, v = rnd((1, 1, 5, 3), 13), rnd((1, 1, 1, 3), 14), rnd((1, 1, 1, 3), 15)
    do = rnd((1, 1, 5, 3), 16)
    dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, False)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    assert np.max(np.abs(dv[0, 0, 0] - do[0, 0].sum(axis=0))) < 1e-12


def test_key_gradients_sum_to_zero():
    # adding one vector c to every key adds q_i . c to all visible scores of row
    # i, which the softmax ignores: the key gradients of a head sum to zero
    for causal in (False, True):
        q, k, v = rnd((2, 4, 7, 5), 17), rnd((2, 2, 9, 5), 18), rnd((2, 2, 9, 5), 19)
        do = rnd((2, 4, 7, 5), 20)
        _, dk, _ = oracle.attention_bwd_fp64(q, k, v, do, causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12


def test_rowsum_identity_used_by_recomputing_backwards():
    # rowsum(P * dP) equals rowsum(dO * O): the per-row term a recomputing
    # backward takes from the forward's output
    q, k, v = rnd((1, 2, 6, 4), 21), rnd((1, 2, 8, 4), 22), rnd((1, 2, 8, 4), 23)
    do = rnd((1, 2, 6, 4), 24)
    o, _ = oracle.attention_fp64(q, k, v, True, threads=1)
    p = oracle.attention_probs_fp64(q, k, True)
    dp = do @ np.swapaxes(v, -1, -2)
    assert np.max(np.abs((p * dp).sum(-1) - (do * o).sum(-1))) < 1e-12


def test_gqa_equals_mha_with_repeated_heads_summed():
    q, k, v = rnd((1, 4, 6, 3), 25), rnd((1, 2, 6, 3), 26), rnd((1, 2, 6, 3), 27)
    do = rnd((1, 4, 6, 3), 28)
    dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, True)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_bwd_fp64(q, kr, vr, do, True)
    assert np.max(np.abs(dq - dq2)) < 1e-12
    assert np.max(np.abs(dk - dk2.reshape(1, 2, 2, 6, 3).sum(axis=2))) < 1e-12
    assert np.max(np.abs(dv - dv2.reshape(1, 2, 2, 6, 3).sum(axis=2))) < 1e-12


def test_head_selection_equals_full_evaluation():
    q, k, v = rnd((2, 4, 5, 3), 29), rnd((2, 2, 5, 3), 30), rnd((2, 2, 5, 3), 31)
    do = rnd((2, 4, 5, 3), 32)
    full = oracle.attention_bwd_fp64(q, k, v, do, True)
    part = oracle.attention_bwd_fp64(q, k, v, do, True, heads=[(1, 2), (1, 3)])
    assert np.array_equal(part[0][1, 2:], full[0][1, 2:]) and np.all(part[0][0] == 0)
    assert np.max(np.abs(part[1][1, 1] - full[1][1, 1])) < 1e-12


# ---- planted mistakes ------------------------------------------------------------

def _mutant(kind):
    def run(q, k, v, do, causal):
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        tau = 1.0 / math.sqrt(d)
        n_vis = np.array([visible_keys(i, Sq, Sk, causal and kind != "no_mask") for i in range(Sq)])
        vis = np.arange(Sk)[None, :] < n_vis[:, None]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                kvh = h // G
                s = np.where(vis, q[b, h] @ k[b, kvh].T * tau, -np.inf)
                e = np.where(vis, np.exp(s - s.max(axis=1)[:, None]), 0)
                p = e / e.sum(axis=1)[:, None]
                pv = p.T @ do[b, h]
                dv[b, kvh] += pv[::-1] if kind == "dv_reversed" else pv
                dp = do[b, h] @ v[b, kvh].T
                ds = p * (dp - (p * dp).sum(axis=1)[:, None]) if kind != "no_rowsum" else p * dp
                if kind == "p_for_ds":
                    ds = p
                t = tau if kind != "no_scale" else 1.0
                dq[b, h] = t * (ds @ k[b, kvh])
                dk[b, kvh] += t * (ds.T @ (q[b, h] if kind != "dk_uses_do" else do[b, h]))
        return dq, dk, dv
    return run


@pytest.mark.parametrize("kind", ["no_mask", "no_rowsum", "p_for_ds", "no_scale", "dk_uses_do", "dv_reversed"])
def test_planted_backward_mistakes_are_caught(kind):
    run = _mutant(kind)
    caught = False
    B, Hq, Hkv, Sq, Sk, d, causal = 1, 2, 1, 5, 5, 3, True
    q, k, v = rnd((B, Hq, Sq, d), 33), rnd((B, Hkv, Sk, d), 34), rnd((B, Hkv, Sk, d), 35)
    do = rnd((B, Hq, Sq, d), 36)
    got = run(q, k, v, do, causal)
    # central differences of the forward oracle
    h = 1e-6
    for x, g in zip((q, k, v), got):
        for idx in list(np.ndindex(x.shape))[:12]:
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(q, k, v, do, causal)
            x[idx] = keep - h
            lm = _loss(q, k, v, do, causal)
            x[idx] = keep
            caught |= abs((lp - lm) / (2 * h) - g[idx]) > 1e-6
    # the key-gradient sum invariant
    caught |= bool(np.max(np.abs(got[1].sum(axis=2))) > 1e-9)
    assert caught, f"mutant {kind} slipped through"
