"""The library on several streams and inside captured HIP graphs.

Every call is asynchronous on the stream it is given and keeps no state
between calls (the caller owns every buffer, workspaces included), so calls
on different streams may run at once and a captured sequence of calls may be
replayed.  Checked bit for bit against the same calls made eagerly on one
stream: two streams running forward and decode work at the same time, and
graphs of a forward, a backward and a decode step replayed three times with
new inputs copied in and eager work of the program's own between replays."""

import pytest
import torch

import fa_inputs

pytestmark = pytest.mark.gpu


def _fwd_inputs(seed, B=2, Hq=8, Hkv=2, S=700):
    cfg = fa_inputs.FwdConfig("t", "bf16", B, Hq, Hkv, S, S, 128, True)
    return fa_inputs.make_fwd_inputs(cfg, seed=seed, device="cuda")


def _decode_inputs(seed):
    cfg = fa_inputs.DecodeConfig("t", 4, 16, 4, 3000, 128, 8, (3000, 1, 1777, 2048))
    return cfg, fa_inputs.make_decode_inputs(cfg, seed=seed, device="cuda")


def _fwd(gpu, x, stream=None):
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], device="cuda")
    gpu.fa_fwd(x["q"], x["k"], x["v"], o, lse, causal=True, stream=stream)
    return o, lse


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_two_streams_at_once(gpu):
    xs = [_fwd_inputs(seed) for seed in (1, 2)]
    cfg, d = _decode_inputs(3)
    ws = gpu.decode_workspace(cfg.B, cfg.Hq, cfg.d, cfg.num_splits, "cuda")
    print("eager, one stream", flush=True)
    ref = [_fwd(gpu, x) for x in xs]
    o_ref = torch.empty(cfg.B, cfg.Hq, cfg.d, dtype=torch.bfloat16, device="cuda")
    gpu.fa_decode_kvq(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], o_ref, None, seq_lens=d["seq_lens"],
                      num_splits=cfg.num_splits, workspace=ws)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    ws2 = gpu.decode_workspace(cfg.B, cfg.Hq, cfg.d, cfg.num_splits, "cuda")
    o_dec = torch.empty_like(o_ref)
    print("two streams at once", flush=True)
    for _ in range(3):
        with torch.cuda.stream(s1):
            got0 = _fwd(gpu, xs[0])
            gpu.fa_decode_kvq(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], o_dec, None,
                              seq_lens=d["seq_lens"], num_splits=cfg.num_splits, workspace=ws2)
        with torch.cuda.stream(s2):
            got1 = _fwd(gpu, xs[1])
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip((got0, got1), ref):
            assert _same(o, ro) and _same(l, rl)
        assert _same(o_dec, o_ref)


def test_graph_replay(gpu):
    """fa_fwd, fa_bwd and fa_decode_kvq captured in one graph; each of three
    replays, with new inputs copied into the captured buffers and eager calls
    in between, equals the eager result bit for bit."""
    cfg, d = _decode_inputs(5)
    x = _fwd_inputs(6)
    dout = torch.randn(x["q"].shape, device="cuda").to(torch.bfloat16)
    # buffers the graph reads and writes
    q, k, v, do = (t.clone() for t in (x["q"], x["k"], x["v"], dout))
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(gpu.fa_bwd_workspace_size(q.shape[0], q.shape[1], q.shape[2]), dtype=torch.uint8,
                      device="cuda")
    dq_ = d["q"].clone()
    o_dec = torch.empty(cfg.B, cfg.Hq, cfg.d, dtype=torch.bfloat16, device="cuda")
    l_dec = torch.empty(cfg.B, cfg.Hq, device="cuda")
    dws = gpu.decode_workspace(cfg.B, cfg.Hq, cfg.d, cfg.num_splits, "cuda")

    def step(stream=None):
        gpu.fa_fwd(q, k, v, o, lse, causal=True, stream=stream)
        gpu.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, causal=True, workspace=bws, stream=stream)
        gpu.fa_decode_kvq(dq_, d["k"], d["v"], d["k_scale"], d["v_scale"], o_dec, l_dec, seq_lens=d["seq_lens"],
                          num_splits=cfg.num_splits, workspace=dws, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture (kernel attributes set once)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("capturing fa_fwd + fa_bwd + fa_decode_kvq", flush=True)
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    outs = (o, lse, dq, dk, dv, o_dec, l_dec)
    for rep in range(3):
        # new inputs copied into the captured buffers
        nx = _fwd_inputs(10 + rep)
        for dst, src in ((q, nx["q"]), (k, nx["k"]), (v, nx["v"])):
            dst.copy_(src)
        do.copy_(torch.randn(do.shape, device="cuda").to(torch.bfloat16))
        dq_.copy_(torch.randn(dq_.shape, device="cuda").to(torch.bfloat16))
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        step()  # the same calls made eagerly on the same buffers
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV", "decode O", "decode LSE"), got, outs):
            assert _same(a, b), f"replay {rep}: {name} differs from the eager call"
