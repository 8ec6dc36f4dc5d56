"""GPU parity at the largest sizes the boundary accepts.

Every kernel addresses one (batch, head) slice through a buffer resource with
32-bit byte offsets, and the validators accept a slice only while it spans
less than 2^31 bytes.  These cases put a slice at that limit and check the rows
that sit at its far end, where an offset computed in too narrow a type or a
range check off by one would show first:

* prefill, bf16, d = 128: K and V slices of 8,388,607 rows (2^31 - 256 bytes),
  causal and not, GQA 2/1, 130 query rows (a ragged tile);
* int8-KV decode: a 16,777,215-token cache slice (2^31 - 128 bytes of codes),
  64 splits;
* quantise-on-append into the last 100 slots of a cache of that length.

A few keys are made to dominate the softmax, at the far end of the slice and
in the middle, so that the outputs depend on those rows and not only on the
average of millions of N(0, 1) values; the LSE checks every visible key.  The
oracle runs in float64 on the host (tens of GB of host memory; about a minute).
"""

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3
SK_MAX = (1 << 31) // 256 - 1  # bf16 rows of 128 elements: the slice spans 2^31 - 256 bytes
L_MAX = (1 << 31) // 128 - 1   # int8 codes of 128 elements: 2^31 - 128 bytes


@pytest.mark.timeout(900)
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_largest_slice(gpu, causal):
    cfg = fa_inputs.FwdConfig("t", "bf16", 1, 2, 1, 130, SK_MAX, 128, causal)
    print(f"fa_fwd largest slice Sk={SK_MAX} causal={causal}", flush=True)
    x = fa_inputs.make_fwd_inputs(cfg, seed=21, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    # every query row has 4 on channel 0; two keys are that channel alone: 80,
    # 200 rows before the end (visible to every row, causal or not; score 28.3),
    # and 120, the very last key (score 42.4; causal: visible to the last query
    # row only).  The other keys' scores are about N(0, 1), log-sum-exp 16.5.
    q[..., 0] = 4.0
    for t, val in ((SK_MAX - 200, 80.0), (SK_MAX - 1, 120.0)):
        k[0, 0, t] = 0.0
        k[0, 0, t, 0] = val
    o = torch.full((1, 2, 130, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 2, 130), float("nan"), device="cuda")
    gpu.fa_fwd(q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()
    rows = [0, 63, 64, 128, 129]
    ro, rl = oracle.attention_fp64(q.cpu(), k.cpu(), v.cpu(), causal, rows=rows)
    og = o[:, :, rows].double().cpu().numpy()
    lg = lse[:, :, rows].double().cpu().numpy()
    assert float(np.max(np.abs(og - ro))) <= TOL_O
    assert float(np.max(np.abs(lg - rl))) <= TOL_LSE
    # the planted keys decide the outputs: row 0 is (almost) the last key's V
    # row, or under the causal mask the V row 200 keys before the end
    want = v[0, 0, SK_MAX - 200 if causal else SK_MAX - 1].double().cpu().numpy()
    assert float(np.max(np.abs(ro[0, :, 0] - want))) < 0.05


@pytest.mark.timeout(900)
def test_decode_largest_slice(gpu):
    cfg = fa_inputs.DecodeConfig("t", 1, 4, 1, L_MAX, 128, 64)
    print(f"fa_decode_kvq largest slice L={L_MAX}", flush=True)
    x = fa_inputs.make_decode_inputs(cfg, seed=22, device="cuda")
    # the last token and one in the middle dominate: channel 0 alone, code 127
    # with scale 1.0, against a query component of 3 there (score 33.7 for
    # both; the other tokens' log-sum-exp is about 17.2)
    for t in (L_MAX - 1, L_MAX // 2):
        x["k"][0, 0, t] = 0
        x["k"][0, 0, t, 0] = 127
        x["k_scale"][0, 0, t] = 1.0
    x["q"][..., 0] = 3.0
    o = torch.full((1, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 4), float("nan"), device="cuda")
    ws = gpu.decode_workspace(1, 4, 128, 64)
    gpu.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse,
                      seq_lens=x["seq_lens"], num_splits=64, workspace=ws)
    torch.cuda.synchronize()
    c = {n: x[n].cpu() for n in ("q", "k", "v", "k_scale", "v_scale", "seq_lens")}
    del x
    ro, rl = oracle.decode_fp64(c["q"], c["k"].numpy(), c["k_scale"].numpy(), c["v"].numpy(),
                                c["v_scale"].numpy(), c["seq_lens"].numpy())
    assert float(np.max(np.abs(o.double().cpu().numpy() - ro))) <= TOL_O
    assert float(np.max(np.abs(lse.double().cpu().numpy() - rl))) <= TOL_LSE
    # the two planted tokens carry almost all the weight
    vv = oracle.dequant_int8_fp64(c["v"][0, 0, [L_MAX // 2, L_MAX - 1]].numpy(),
                                  c["v_scale"][0, 0, [L_MAX // 2, L_MAX - 1]].numpy())
    assert float(np.max(np.abs(ro[0, 0] - vv.mean(axis=0)))) < 0.05


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_append_at_the_end_of_the_largest_slice(gpu, fmt):
    T = 100
    cfg = fa_inputs.AppendConfig("t", 1, 1, T, L_MAX, 128, fmt, L_MAX - T)
    print(f"fa_kv_append largest slice L={L_MAX} {fmt}", flush=True)
    x = fa_inputs.make_append_inputs(cfg, seed=23, device="cuda")
    # sentinels before the written range must survive
    x["k_cache"][0, 0, L_MAX - T - 1] = 0x11
    x["v_scale"][0, 0, L_MAX - T - 1] = 7.0
    gpu.fa_kv_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                     positions=x["positions"], kv_format=fmt)
    torch.cuda.synchronize()
    for new, codes, scales in (("k_new", "k_cache", "k_scale"), ("v_new", "v_cache", "v_scale")):
        rc, rs = oracle.quantize_kv_tokhead(x[new].cpu(), fmt)
        gc = x[codes][0, 0, L_MAX - T:].cpu().numpy()
        gs = x[scales][0, 0, L_MAX - T:].cpu().numpy()
        assert np.array_equal(gc.view(np.uint8), rc[0, 0].view(np.uint8))
        assert np.array_equal(gs.view(np.uint16), rs[0, 0].view(np.uint16))
    assert bool((x["k_cache"][0, 0, L_MAX - T - 1] == 0x11).all())
    assert float(x["v_scale"][0, 0, L_MAX - T - 1]) == 7.0


@pytest.mark.timeout(900)
def test_backward_largest_slice(gpu):
    """fa_bwd with K, V, dK and dV slices of 8,388,607 rows and 64 query rows
    (bottom-right causal); all of dQ, dK and dV against the oracle (the backward
    tolerance: 2e-2 of each gradient's largest magnitude, plus 1e-4).

    Two keys at the far end get scores near the log-sum-exp of all the others
    (about 16.5), so they hold about half of the weight: their gradient rows
    are then large and are what the relative bar checks.  (A key that takes
    all of the weight would make the exact gradient cancel to nearly zero,
    leaving only the rounding of the forward's bf16 output in the row term.)"""
    Sq = 64
    cfg = fa_inputs.BwdConfig("t", "bf16", 1, 1, 1, Sq, SK_MAX, 128, True)
    print(f"fa_bwd largest slice Sk={SK_MAX}", flush=True)
    x = fa_inputs.make_bwd_inputs(cfg, seed=24, device="cuda")
    q, k, v, dout = x["q"], x["k"], x["v"], x["dout"]
    q[..., 0] = 4.0
    planted = (SK_MAX - 200, SK_MAX - 1)  # the last key: seen by the last query row only
    for t in planted:
        k[0, 0, t] = 0.0
        k[0, 0, t, 0] = 46.0  # score 4 * 46 / sqrt(128) = 16.3
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, Sq, device="cuda")
    gpu.fa_fwd(q, k, v, o, lse, causal=True)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    gpu.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_fp64(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), True)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        g = got.double().cpu().numpy()
        assert not np.isnan(g).any(), name
        scale = float(np.max(np.abs(ref)))
        err = float(np.max(np.abs(g - ref)))
        print(f"{name}: max err {err:.3g}, max |ref| {scale:.3g}", flush=True)
        assert err <= 2e-2 * scale + 1e-4, name
    # the planted rows carry the largest key gradients, far above the 1e-4 floor
    for ref in (rk, rv):
        assert float(np.max(np.abs(ref[0, 0, list(planted)]))) > 0.5
        assert float(np.max(np.abs(ref[0, 0, list(planted)]))) >= 0.5 * float(np.max(np.abs(ref)))
