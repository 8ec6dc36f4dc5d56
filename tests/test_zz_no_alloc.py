"""fa_decode_kvq_noalloc (the decode entry point that allocates nothing: its
split partials live in the library's fixed per-GPU scratch) against
fa_decode_kvq on the same inputs, through the C ABI: two calls in a row, the
second smaller, each bitwise equal to the allocating entry point (same
kernels, same partial layout) and within the quantised-KV bars of the
oracle.  Also: sizes beyond the scratch are refused before anything runs."""

import ctypes

import numpy as np
import pytest
import torch

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, L, lens, W, seed):
    cfg = fa_inputs.DecodeConfig("t", B, Hq, Hkv, L, 128, 16, tuple(lens), "int8", W)
    xc = fa_inputs.make_decode_inputs(cfg, seed=seed)
    return xc, {k: v.cuda() for k, v in xc.items()}


def _both(fa, x, splits, W):
    B, Hq, d = x["q"].shape
    win = {}
    if W:
        win = dict(k_recent=x["k_recent"], v_recent=x["v_recent"], recent_lens=x["recent_lens"])
    outs = []
    for name in ("fa_decode_kvq", "fa_decode_kvq_noalloc"):
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        print(f"{name} B={B} Hq={Hq} L={x['k'].shape[2]} splits={splits} W={W}", flush=True)
        getattr(fa, name)(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse,
                          seq_lens=x["seq_lens"], num_splits=splits, **win)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


def test_noalloc_matches_the_allocating_entry(gpu):
    # first call: 8 sequences of up to 8192 tokens, 16 splits, a 40-token
    # window (17 partial slots); second call smaller: 3 sequences, 4 splits
    for B, Hq, Hkv, L, lens, W, splits in [(8, 32, 8, 8192, [8192, 1, 5000, 8191, 33, 4096, 0, 7777], 40, 16),
                                           (3, 8, 2, 1000, [1000, 513, 7], 0, 4)]:
        xc, x = _inputs(B, Hq, Hkv, L, lens, W, seed=B + L)
        (o1, l1), (o2, l2) = _both(gpu, x, splits, W)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs from fa_decode_kvq"
        assert torch.equal(l1.isnan(), l2.isnan()) and bool((l1 == l2)[~l1.isnan()].all())
        win = {}
        if W:
            win = dict(k_recent=xc["k_recent"], v_recent=xc["v_recent"], recent_lens=xc["recent_lens"].numpy())
        ro, rl = oracle.decode_fp64(xc["q"], xc["k"].numpy(), xc["k_scale"].numpy(), xc["v"].numpy(),
                                    xc["v_scale"].numpy(), xc["seq_lens"].numpy(), **win)
        og, lg = o2.double().cpu().numpy(), l2.double().cpu().numpy()
        assert float(np.max(np.abs(og - ro))) <= 8e-2
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lg), fin)
        assert float(np.max(np.abs(lg[fin] - rl[fin]), initial=0.0)) <= 1e-3


def test_noalloc_refuses_sizes_beyond_its_scratch(gpu):
    # 64 splits of 64 x 32 query heads need 67.6 MB of partials (> 32 MiB)
    xc, x = _inputs(64, 32, 8, 64, [], 0, seed=1)
    o = torch.empty(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.FaError) as e:
        gpu.fa_decode_kvq_noalloc(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, None, num_splits=64)
    assert e.value.status == gpu.FA_ERR_WORKSPACE
    assert gpu.fa_decode_workspace_size(64, 32, 128, 64) > gpu.FA_DECODE_NOALLOC_MAX_BYTES
