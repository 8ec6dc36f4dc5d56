"""Throughput of the exact tiled attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--extra all|none|NAME,...] [--no-cpu-baseline]

A step is one call of the hot path over one batch of synthetic input already
resident in HBM.  The headline workload is the largest prefill configuration:
causal bf16 long-context grouped-query prefill, B=1, Hq=32, Hkv=8, S=16384,
d=128, 1 % of the key rows scaled by 8, with LSE output; its TFLOP/s counts
4*d flops per visible (query, key) pair (S*(S+1)/2 pairs per head under the
causal mask).  The other workloads are timed the same way and reported under
"workloads": the other four configurations (fp32 S=128, causal bf16 B=4 H=16
S=2048, fp8 B=8 H=16 S=4096, int8-KV split decode), the backward of the two
causal bf16 workloads in TFLOP/s (10 d flops per visible pair), the fp8
prefill on 64-row block-scaled, rotated codes, the fp8 prefill with bf16
probabilities, fp8-KV decode, the decode with a bf16 residual window, the
quantise-on-append of a 4096-token chunk and the fp8 block quantiser in GB/s
of the bytes the method must move.

Timing uses HIP events on the stream the kernels are launched on (torch's
current stream), bracketed by device synchronisations, after at least W
untimed calls and at least 0.3 s of untimed work, so the clocks have settled.
"ms_per_call" is the mean over the timed region; a second pass with an event
pair around every call gives "ms_median" and "ms_min".  For each of the five
configurations the float64 oracle is then timed on this host's cores over a
bounded sample (whole heads, or whole batch entries for decode), reported as
"cpu_baseline" in the workload's unit, and the GPU outputs of that sample are
compared with it ("max_abs_err").  Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs  # noqa: E402

METRIC = "attention fwd TFLOP/s and % MFMA peak; decode KV GB/s and % HBM peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk/CU x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_gqa32x8_s16384_causal_outlier"
PROFILES = os.path.join(ROOT, "profiles")


# ---- algorithmic work ---------------------------------------------------------

def visible_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """(query, key) pairs the mask leaves visible in one head."""
    if not causal:
        return Sq * Sk
    # row i sees min(Sk, max(0, i + Sk - Sq + 1)) keys
    off = Sk - Sq
    return sum(min(Sk, max(0, i + off + 1)) for i in range(Sq))


def fwd_flops(cfg) -> int:
    """2*d flops for S = Q K^T plus 2*d for O = P V, per visible pair per head."""
    return 4 * cfg.d * visible_pairs(cfg.Sq, cfg.Sk, cfg.causal) * cfg.B * cfg.Hq


def fwd_hbm_bytes(cfg) -> int:
    """Compulsory HBM bytes of one prefill: Q, K, V read once, O (and LSE) written."""
    es = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}[cfg.dtype]
    oes = 4 if cfg.dtype == "f32" else 2
    q = cfg.B * cfg.Hq * cfg.Sq * cfg.d * es
    kv = 2 * cfg.B * cfg.Hkv * cfg.Sk * cfg.d * es
    o = cfg.B * cfg.Hq * cfg.Sq * cfg.d * oes
    lse = cfg.B * cfg.Hq * cfg.Sq * 4
    return q + kv + o + lse


def decode_bytes(cfg) -> int:
    """KV bytes = 2 * layers * batch * tokens * kv_heads * head_dim * bytes_per_elem
    with one layer and 1-byte codes (int8 or fp8), plus the per-token fp16 scales
    of K and V, the bf16 residual window's keys and values when there is one,
    the bf16 query, the bf16 output and the float32 LSE."""
    kv = 2 * 1 * cfg.B * cfg.L * cfg.Hkv * cfg.d * 1
    scales = 2 * cfg.B * cfg.Hkv * cfg.L * 2
    window = 2 * cfg.B * cfg.Hkv * cfg.W * cfg.d * 2
    q = cfg.B * cfg.Hq * cfg.d * 2
    o = cfg.B * cfg.Hq * cfg.d * 2
    lse = cfg.B * cfg.Hq * 4
    return kv + scales + window + q + o + lse


def bwd_flops(cfg) -> int:
    """The backward's five products per visible pair: S recomputed (2d), dP = dO V^T
    (2d), dV = P^T dO (2d), dQ = dS K (2d), dK = dS^T Q (2d): 10 d flops, 2.5x the
    forward.  Recomputations beyond these (S and dP are formed in both the dK/dV
    and the dQ pass here) are not counted."""
    return 10 * cfg.d * visible_pairs(cfg.Sq, cfg.Sk, cfg.causal) * cfg.B * cfg.Hq


def append_bytes(cfg) -> int:
    """Quantise-on-append: the bf16 key and value rows read once, their 1-byte
    codes and fp16 per-row scales written once."""
    rows = cfg.B * cfg.H * cfg.T
    return 2 * rows * cfg.d * 2 + 2 * (rows * cfg.d + rows * 2)


def bwd_hbm_bytes(cfg) -> int:
    """Compulsory HBM bytes of one backward: Q, K, V, O, dO and LSE read once,
    dQ, dK, dV written once."""
    q = cfg.B * cfg.Hq * cfg.Sq * cfg.d * 2
    kv = cfg.B * cfg.Hkv * cfg.Sk * cfg.d * 2
    return 3 * q + 2 * kv + cfg.B * cfg.Hq * cfg.Sq * 4 + q + 2 * kv


def quant_bytes(cfg) -> int:
    """Block quantiser over Q, K and V: bf16 rows read once, 1-byte codes and one
    float32 scale per 64-row block written once (the 128 signs are not counted)."""
    n = cfg.B * cfg.H * cfg.S * cfg.d
    blocks = cfg.B * cfg.H * ((cfg.S + 63) // 64)
    return 3 * (n * 2 + n + blocks * 4)


def algorithmic_bytes(cfg) -> int:
    if isinstance(cfg, fa_inputs.QuantConfig):
        return quant_bytes(cfg)
    if isinstance(cfg, fa_inputs.BwdConfig):
        return bwd_hbm_bytes(cfg)
    if isinstance(cfg, fa_inputs.DecodeConfig):
        return decode_bytes(cfg)
    if isinstance(cfg, fa_inputs.AppendConfig):
        return append_bytes(cfg)
    return fwd_hbm_bytes(cfg)


def launches_per_call(cfg) -> int:
    """Launches of the workload's dominant kernel in one call (the quantiser
    runs once per tensor: Q, K and V)."""
    return 3 if isinstance(cfg, fa_inputs.QuantConfig) else 1


def workload(name):
    for table in (fa_inputs.CONFIGS, fa_inputs.BWD_CONFIGS, fa_inputs.KV_CONFIGS, fa_inputs.FP8_VARIANT_CONFIGS,
                  fa_inputs.SOFT_EXP2_CONFIGS, fa_inputs.NO_LSE_CONFIGS, fa_inputs.BWD_VARIANT_CONFIGS):
        if name in table:
            return table[name]
    raise KeyError(name)



# ---- GPU timing ---------------------------------------------------------------

WARMUP_SECONDS = 0.3


def _time_region(fn, steps, warmup):
    """Mean per-call time (ms) of `steps` calls after at least `warmup` untimed
    calls and at least WARMUP_SECONDS of untimed work (the clocks settle first)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARMUP_SECONDS:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def _time_each(fn, steps):
    """Per-call times (ms) from an event pair around every call, on the launch
    stream; run right after _time_region, so the clocks are settled."""
    import torch

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))


class Runner:
    """One workload on the GPU: run() enqueues one call; check(budget_s), when
    given, times the float64 oracle on a bounded sample of the same inputs and
    compares the GPU outputs of that sample with it."""

    def __init__(self, run, check=None):
        self.run = run
        self.check = check


def _cores():
    return len(os.sched_getaffinity(0))


def _cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _fwd_oracle_check(cfg, x, o, lse, budget_s):
    """The oracle over whole (batch, head) pairs of a prefill workload, as many
    as fit the budget (whole passes repeated when the workload is smaller).
    The inputs are upcast (fp8: decoded and descaled) to float64 once, before
    the timed part."""
    import numpy as np

    import oracle
    from oracle.e4m3 import e4m3_decode

    if cfg.dtype == "fp8":
        qf = e4m3_decode(x["q"].cpu()) * x["q_scale"]
        kf = e4m3_decode(x["k"].cpu()) * x["k_scale"]
        vf = e4m3_decode(x["v"].cpu()) * x["v_scale"]
    else:
        qf, kf, vf = (x[n].cpu().double().numpy() for n in ("q", "k", "v"))
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy() if lse is not None else None
    cores = _cores()
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    n = min(len(heads), cores)
    done, elapsed, err_o, err_l, checked = 0, 0.0, 0.0, 0.0, 0
    while done == 0 or elapsed < budget_s * 0.85:
        start = done % len(heads)
        part = heads[start:start + n]
        t0 = time.perf_counter()
        ro, rl = oracle.attention_fp64(qf, kf, vf, cfg.causal, cfg.scale, heads=part, threads=cores)
        elapsed += time.perf_counter() - t0
        if done < len(heads):  # first pass: compare
            bi = [b for b, _ in part]
            hi = [h for _, h in part]
            err_o = max(err_o, float(np.max(np.abs(og[bi, hi] - ro[bi, hi]))))
            if lg is not None:
                fin = np.isfinite(rl[bi, hi])
                err_l = max(err_l, float(np.max(np.abs(lg[bi, hi][fin] - rl[bi, hi][fin]), initial=0.0)))
            checked += len(part)
        done += len(part)
        # stop before a chunk that would overrun the budget
        if elapsed / done * (done + n) > budget_s:
            break
    flops = fwd_flops(cfg) * done / len(heads)
    if done <= len(heads):
        sample = f"{done} of {len(heads)} (batch, head) pairs"
    else:
        sample = f"{done / len(heads):.1f} passes over all {len(heads)} (batch, head) pairs"
    cpu = {"value": flops / elapsed / 1e9, "unit": "GFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{sample} of {cfg.name}, float64 numpy two-pass, {elapsed:.1f} s wall",
           "cpu_model": _cpu_model()}
    err = {"O": err_o, "LSE": err_l if lg is not None else None,
           "sample": f"{checked} of {len(heads)} (batch, head) pairs, every row"}
    return cpu, err


def _decode_oracle_check(cfg, x, o, lse, budget_s):
    """The oracle over whole batch entries of a decode workload (every query
    head of the entry), as many as fit the budget; the oracle dequantises the
    codes it reads.  GB/s of the entries' share of the algorithmic bytes."""
    import numpy as np

    import oracle

    cores = _cores()
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    done, elapsed, err_o, err_l = 0, 0.0, 0.0, 0.0
    order = [0, cfg.B - 1] + list(range(1, cfg.B - 1))
    per_entry = decode_bytes(cfg) / cfg.B
    while done < cfg.B:
        b = order[done]
        sub = {n: x[n][b:b + 1].cpu() for n in ("q", "k", "v", "k_scale", "v_scale", "seq_lens")}
        t0 = time.perf_counter()
        ro, rl = oracle.decode_fp64(sub["q"], sub["k"].numpy(), sub["k_scale"].numpy(), sub["v"].numpy(),
                                    sub["v_scale"].numpy(), sub["seq_lens"].numpy(), scale=cfg.scale,
                                    threads=cores, kv_format=cfg.kv_format)
        elapsed += time.perf_counter() - t0
        err_o = max(err_o, float(np.max(np.abs(og[b:b + 1] - ro))))
        fin = np.isfinite(rl)
        err_l = max(err_l, float(np.max(np.abs(lg[b:b + 1][fin] - rl[fin]), initial=0.0)))
        done += 1
        if elapsed / done * (done + 1) > budget_s:
            break
    cpu = {"value": per_entry * done / elapsed / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"{done} of {cfg.B} batch entries of {cfg.name} (all {cfg.Hq} heads each), float64 numpy, "
                     f"{elapsed:.1f} s wall", "cpu_model": _cpu_model()}
    err = {"O": err_o, "LSE": err_l, "sample": f"{done} of {cfg.B} batch entries, every head"}
    return cpu, err


def _fwd_runner(cfg, seed=0, p_bf16=False, soft_exp2=False):
    import torch

    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_fwd_inputs(cfg, seed=seed, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.bfloat16}[cfg.dtype]
    o = torch.empty(q.shape, dtype=odt, device="cuda")
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Sq, dtype=torch.float32, device="cuda") if cfg.lse else None
    ds = (x.get("q_scale", 1.0), x.get("k_scale", 1.0), x.get("v_scale", 1.0))

    def run():
        fa.fa_fwd(q, k, v, o, lse, causal=cfg.causal, softmax_scale=cfg.scale,
                  q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], p_bf16=p_bf16, soft_exp2=soft_exp2)

    return Runner(run, lambda budget: _fwd_oracle_check(cfg, x, o, lse, budget))


def _quantise_block_fp8(fa, x, signs):
    """q, k, v (bf16 on the GPU) -> codes and 64-row block scales, Q and K rotated
    when signs are given, by the library's quantiser."""
    import torch

    out = {}
    for n in ("q", "k", "v"):
        t = x[n]
        codes = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
        sc = torch.empty(t.shape[0], t.shape[1], (t.shape[2] + 63) // 64, dtype=torch.float32, device=t.device)
        fa.fa_fp8_quantize(t, codes, sc, signs if n != "v" else None)
        out[n], out[n + "_bs"] = codes, sc
    return out


def _fp8_block_runner(cfg, seed=0):
    import dataclasses

    import torch

    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_fwd_inputs(dataclasses.replace(cfg, dtype="bf16"), seed=seed, device="cuda")
    signs = fa_inputs.make_rotation_signs(cfg.d, seed, "cuda") if cfg.rotate else None
    c = _quantise_block_fp8(fa, x, signs)
    del x
    q, k, v = (c[n].view(torch.float8_e4m3fn) for n in ("q", "k", "v"))
    bds = (c["q_bs"], c["k_bs"], c["v_bs"])
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Sq, dtype=torch.float32, device="cuda")

    def run():
        fa.fa_fwd(q, k, v, o, lse, causal=cfg.causal, softmax_scale=cfg.scale, block_descales=bds)

    return Runner(run)


def _quant_runner(cfg, seed=0):
    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_quant_inputs(cfg, seed=seed, device="cuda")

    def run():
        _quantise_block_fp8(fa, x, x["signs"])

    return Runner(run)


def _decode_runner(cfg, seed=0):
    import torch

    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_decode_inputs(cfg, seed=seed, device="cuda")
    o = torch.empty(cfg.B, cfg.Hq, cfg.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(cfg.B, cfg.Hq, dtype=torch.float32, device="cuda")
    ws = fa.decode_workspace(cfg.B, cfg.Hq, cfg.d, cfg.num_splits, window=cfg.W > 0)
    win = {}
    if cfg.W > 0:
        win = {"k_recent": x["k_recent"], "v_recent": x["v_recent"], "recent_lens": x["recent_lens"]}

    def run():
        fa.fa_decode_kvq(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], o, lse,
                         seq_lens=x["seq_lens"], num_splits=cfg.num_splits,
                         softmax_scale=cfg.scale, workspace=ws, kv_format=cfg.kv_format, **win)

    check = None if cfg.W > 0 else (lambda budget: _decode_oracle_check(cfg, x, o, lse, budget))
    return Runner(run, check)


def _bwd_runner(cfg, seed=0):
    import torch

    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_bwd_inputs(cfg, seed=seed, device="cuda")
    q, k, v, dout = x["q"], x["k"], x["v"], x["dout"]
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.Hq, cfg.Sq, dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, causal=cfg.causal, softmax_scale=cfg.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(cfg.B, cfg.Hq, cfg.Sq), dtype=torch.uint8, device="cuda")
    pingpong = isinstance(cfg, fa_inputs.PingPongBwdConfig)

    def run():
        fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=cfg.causal, softmax_scale=cfg.scale, workspace=ws,
                  wave_pingpong=pingpong)

    return Runner(run)


def _append_runner(cfg, seed=0):
    import tiled_exact_attention_fa_amd as fa

    x = fa_inputs.make_append_inputs(cfg, seed=seed, device="cuda")

    def run():  # every call writes the same chunk to the same slots
        fa.fa_kv_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                        positions=x["positions"], kv_format=cfg.kv_format)

    return Runner(run)


# the files that hold each kernel family's device code
KERNEL_SOURCES = {
    "fwd16": ["fa_fwd_mfma.hip", "fa_fwd_common.hpp", "fa_device.hpp"],
    "fwd8": ["fa_fwd_fp8.hip", "fa_fwd_common.hpp", "fa_device.hpp"],
    "decode": ["fa_decode.hip", "fa_device.hpp"],
    "append": ["fa_kv_append.hip", "fa_device.hpp"],
    "bwd": ["fa_bwd.hip", "fa_device.hpp"],
    "quant": ["fa_fp8_quant.hip", "fa_device.hpp"],
}


def kernel_family(cfg) -> str:
    if isinstance(cfg, fa_inputs.QuantConfig):
        return "quant"
    if isinstance(cfg, fa_inputs.DecodeConfig):
        return "decode"
    if isinstance(cfg, fa_inputs.AppendConfig):
        return "append"
    if isinstance(cfg, fa_inputs.BwdConfig):
        return "bwd"
    return "fwd8" if cfg.dtype == "fp8" else "fwd16"


def source_digest(family: str) -> str:
    """Hash of one kernel family's sources, to tie stored counter readings to
    the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_exact_attention_fa_amd", "csrc")
    for n in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(name: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current sources of the workload's kernels; else None."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(name)
    if not ent or ent.get("source_digest") != source_digest(kernel_family(workload(name))):
        return None
    return ent.get("bytes_per_launch")


def _runner(cfg):
    """The Runner of any workload configuration."""
    if isinstance(cfg, fa_inputs.DecodeConfig):
        return _decode_runner(cfg)
    if isinstance(cfg, fa_inputs.AppendConfig):
        return _append_runner(cfg)
    if isinstance(cfg, fa_inputs.QuantConfig):
        return _quant_runner(cfg)
    if isinstance(cfg, fa_inputs.BwdConfig):
        return _bwd_runner(cfg)
    if isinstance(cfg, fa_inputs.Fp8BlockConfig):
        return _fp8_block_runner(cfg)
    return _fwd_runner(cfg, p_bf16=isinstance(cfg, fa_inputs.Fp8PBf16Config),
                       soft_exp2=isinstance(cfg, fa_inputs.SoftExp2Config))


def work_and_unit(cfg):
    """Algorithmic work of one call and the unit its rate is given in."""
    if isinstance(cfg, (fa_inputs.DecodeConfig, fa_inputs.AppendConfig, fa_inputs.QuantConfig)):
        return algorithmic_bytes(cfg), "GB/s"
    if isinstance(cfg, fa_inputs.BwdConfig):
        return bwd_flops(cfg), "TFLOP/s"
    return fwd_flops(cfg), "TFLOP/s"


def measure(name, steps, warmup, check_budget=0.0, clock=False):
    """Times one workload; with check_budget > 0 and an oracle check for it,
    also the CPU baseline and the max error on the oracle's sample; with
    clock, also the gfx clock and socket power observed while it runs (after
    the timed region)."""
    cfg = workload(name)
    import torch

    r = _runner(cfg)
    ms, wall = _time_region(r.run, steps, warmup)
    each = _time_each(r.run, steps)
    med, mn = each[len(each) // 2], each[0]
    if isinstance(cfg, (fa_inputs.DecodeConfig, fa_inputs.AppendConfig, fa_inputs.QuantConfig)):
        work = algorithmic_bytes(cfg)
        gbs = work / (ms * 1e-3) / 1e9
        res = {"unit": "GB/s", "value": gbs, "bytes_per_call": work,
               "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": gbs / PEAK_HBM_GBS, "traffic": stored_traffic(name)}}
    else:
        work = bwd_flops(cfg) if isinstance(cfg, fa_inputs.BwdConfig) else fwd_flops(cfg)
        tf = work / (ms * 1e-3) / 1e12
        # a contraction is priced against the dense MFMA peak of its own input type
        peak = {"f32": PEAK_F32_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(cfg.dtype, PEAK_BF16_TFLOPS)
        res = {"unit": "TFLOP/s", "value": tf, "flops_per_call": work,
               "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                            "frac": tf / peak, "traffic": stored_traffic(name)}}
        if cfg.dtype == "fp8":
            # the prefill target is stated against the bf16 peak for every input type
            res["frac_of_bf16_peak"] = tf / PEAK_BF16_TFLOPS
    res.update({"ms_per_call": ms, "ms_median": med, "ms_min": mn, "wall_s": wall})
    if clock:
        res["observed"] = observed_clock(r.run, ms)
    if check_budget > 0 and r.check is not None:
        res["cpu_baseline"], res["max_abs_err"] = r.check(check_budget)
    del r
    torch.cuda.empty_cache()
    return res


# ---- HBM traffic from rocprofv3 counters ------------------------------------

def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device copy of nbytes (read nbytes, write nbytes), for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)  # an elementwise kernel: reads x once, writes y once
    torch.cuda.synchronize()


def stream_ceiling(nbytes: int = 4_363_132_928, steps: int = 10):
    """Practical HBM ceilings from vendor kernels on a buffer the size of the
    int8 decode workload's algorithmic bytes: a read-only reduction (max over
    int64 words: every byte read once, nothing written of note) and a copy
    (read and write).  One markdown row each."""
    import torch

    n = nbytes // 8
    x = torch.randint(0, 1 << 30, (n,), dtype=torch.int64, device="cuda")
    y = torch.empty_like(x)
    print("| kernel | bytes moved per call | ms per call | GB/s |")
    print("|---|---|---|---|")
    rows = [("read: torch.amax over int64 words", lambda: torch.amax(x), 8 * n),
            ("read: torch.sum over int64 words", lambda: torch.sum(x), 8 * n),
            ("copy: y.copy_(x)", lambda: y.copy_(x), 16 * n)]
    for name, fn, moved in rows:
        ms, _ = _time_region(fn, steps, 3)
        print(f"| {name} | {moved} | {ms:.4f} | {moved / (ms * 1e-3) / 1e9:.0f} |", flush=True)
    del x, y
    torch.cuda.empty_cache()


def _pmc_per_dispatch(csv_dir: str, counter: str, kernel_substr: str):
    import csv
    import glob

    vals = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} under {csv_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize_pmc(a):
    """Turns four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the
    workload, and of the copy calibration) into bytes per launch, records them
    in profiles/hbm_traffic.json with the kernel-source digest, and prints a
    markdown summary."""
    nbytes = a.calib_bytes
    cf, _ = _pmc_per_dispatch(a.calib_fetch, "FETCH_SIZE", a.calib_kernel)
    cw, _ = _pmc_per_dispatch(a.calib_write, "WRITE_SIZE", a.calib_kernel)
    f_scale = nbytes / (cf * 1024.0)
    w_scale = nbytes / (cw * 1024.0)
    wf, nf = _pmc_per_dispatch(a.pmc_fetch, "FETCH_SIZE", a.kernel)
    ww, nw = _pmc_per_dispatch(a.pmc_write, "WRITE_SIZE", a.kernel)
    fetch = wf * 1024.0 * f_scale
    write = ww * 1024.0 * w_scale
    cfg = workload(a.workload)
    algo = algorithmic_bytes(cfg) // launches_per_call(cfg)  # per launch, like the counters
    path = os.path.join(PROFILES, "hbm_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[a.workload] = {"kernel": a.kernel, "bytes_per_launch": fetch + write, "fetch_bytes": fetch,
                        "write_bytes": write, "algorithmic_bytes": algo, "fetch_scale": f_scale,
                        "write_scale": w_scale, "source_digest": source_digest(kernel_family(cfg))}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(f"| {a.workload} | {a.kernel} | {nf} | {wf:.0f} | {ww:.0f} | {f_scale:.4f} | {w_scale:.4f} | "
          f"{fetch / 1e6:.1f} | {write / 1e6:.1f} | {algo / 1e6:.1f} | {(fetch + write) / algo:.3f} |")


# ---- kernel trace against the bench's own per-call times ---------------------

def _kernel_label(name: str) -> str:
    """Readable kernel name: the trace gives the demangled form, or the
    mangled one when the demangler does not know a template argument
    (bf16: DF16b); template arguments are spelled out either way."""
    import re

    if name.startswith("_ZN2fa"):
        m = re.match(r"_ZN2fa\d+(\w+?)I(.*)EEvN", name)
        if not m:
            return name
        args = re.findall(r"DF16b|DF16_|Li(-?\d+)E|Lb(\d)E", m.group(2))
        toks = re.finditer(r"DF16b|DF16_|Li(-?\d+)E|Lb(\d)E", m.group(2))
        out = []
        for t in toks:
            g = t.group(0)
            out.append("bf16" if g == "DF16b" else "f16" if g == "DF16_" else (t.group(1) or t.group(2)))
        del args
        return f"{m.group(1)}<{', '.join(out)}>"
    label = name.replace("void ", "").split("(")[0].replace("fa::", "")
    # the tracer's demangler garbles some template argument lists (a bool
    # pack comes out as "<bool _Accum, bool, E>"): drop those rather than
    # print them
    if "_Accum" in label:
        label = label.split("<")[0]
    return label


def summarize_trace(trace_csv: str, bench_json: str):
    """Markdown table of a rocprofv3 --kernel-trace run of this script: the
    library's dispatches come in one contiguous block per workload (other
    kernels, the input generators', separate them; setup blocks of fewer than
    five dispatches, like the quantiser run before the block-scaled prefill,
    are skipped), taken in the order the script ran the workloads; for each
    kernel of a block its dispatch count and duration, and the bench's own
    mean and median time per call from the same run."""
    import csv
    import statistics

    with open(bench_json) as f:
        line = [ln for ln in f.read().splitlines() if ln.startswith("{")][-1]
    out = json.loads(line)
    order = [out["config"]["workload"]] + list(out["workloads"])
    per_call = {out["config"]["workload"]: (out["ms_per_step"], out.get("ms_median"))}
    for n, w in out["workloads"].items():
        per_call[n] = (w.get("ms_per_call"), w.get("ms_median"))
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                         int(r["Grid_Size_X"])))
    rows.sort()
    blocks, cur = [], []
    for t0, t1, name, grid in rows:
        if "fa::" in name or name.startswith("_ZN2fa"):
            cur.append((_kernel_label(name), grid, t1 - t0))
        elif cur:
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    blocks = [b for b in blocks if len(b) >= 5]
    print("| workload | kernel | grid threads | dispatches | avg us | median us | min us | bench ms/call (mean, median) |")
    print("|---|---|---|---|---|---|---|---|")
    for wl, b in zip(order, blocks):
        kinds = {}
        for short, grid, ns in b:
            kinds.setdefault((short, grid), []).append(ns)
        for (short, grid), ns in kinds.items():
            ms = per_call.get(wl, (None, None))
            bt = f"{ms[0]:.4f}, {ms[1]:.4f}" if ms[0] is not None else "-"
            print(f"| {wl} | {short} | {grid} | {len(ns)} | {statistics.mean(ns) / 1e3:.1f} | "
                  f"{statistics.median(ns) / 1e3:.1f} | {min(ns) / 1e3:.1f} | {bt} |")


# ---- instruction counters ----------------------------------------------------

def summarize_counters(dirs: str, kernel: str, workload_name: str):
    """One markdown row of rocprofv3 --pmc runs (comma-separated output
    directories) of one workload: each counter's mean per dispatch of the
    kernels whose name contains `kernel`, and the figures derived from them
    when present.  Kernel cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8
    XCDs); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles);
    co-exec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; per-MFMA
    counts divide by SQ_INSTS_MFMA (VALU excluding the MFMAs themselves)."""
    means, n_disp = {}, 0
    for d in dirs.split(","):
        import glob

        counters = set()
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            import csv

            with open(path) as f:
                for r in csv.DictReader(f):
                    counters.add(r["Counter_Name"])
        for c in sorted(counters):
            try:
                means[c], n = _pmc_per_dispatch(d, c, kernel)
                n_disp = max(n_disp, n)
            except SystemExit:
                pass
    cyc = means.get("GRBM_GUI_ACTIVE", 0.0) / 8
    mf = means.get("SQ_INSTS_MFMA", 0.0)
    parts = [workload_name, str(n_disp), f"{cyc:.3g}" if cyc else "-"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in means and cyc:
        parts.append(f"{100 * means['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cyc):.1f} %")
    else:
        parts.append("-")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in means and means.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        parts.append(f"{100 * means['SQ_VALU_MFMA_COEXEC_CYCLES'] / means['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} %")
    else:
        parts.append("-")
    for key, sub in (("SQ_INSTS_VALU", mf), ("SQ_INSTS_VALU_TRANS_F32", 0.0), ("SQ_INSTS_LDS", 0.0)):
        parts.append(f"{(means[key] - sub) / mf:.2f}" if key in means and mf else "-")
    if "SQ_LDS_BANK_CONFLICT" in means and means.get("SQ_LDS_IDX_ACTIVE"):
        parts.append(f"{100 * means['SQ_LDS_BANK_CONFLICT'] / means['SQ_LDS_IDX_ACTIVE']:.2f} %")
    else:
        parts.append("-")
    print("| " + " | ".join(parts) + " |")
    print("raw means per dispatch: " + ", ".join(f"{k}={v:.4g}" for k, v in sorted(means.items())))


def summarize_memory(dirs: str, kernel: str, label: str):
    """Memory-pipeline figures of rocprofv3 --pmc runs (comma-separated output
    directories) for the kernels whose name contains `kernel`, means over
    their dispatches: texture-address (TA) busy share of all CU cycles and the
    share of that stalled by the L1 (TCP); average L2-to-memory read latency
    (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ) and reads in flight; DRAM credit
    stalls and L2 busy per channel-cycle (128 channels); L1 pending-stall share;
    the wave-state split (waiting on a dependency / ready but not issued /
    issuing).  Kernel cycles = GRBM_GUI_ACTIVE / 8."""
    import csv
    import glob

    per = {}
    for d in dirs.split(","):
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if kernel not in r["Kernel_Name"]:
                        continue
                    key = (d, r["Dispatch_Id"])
                    per.setdefault(key, {})
                    per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatches of {kernel!r} under {dirs}")
    sums, cnt = {}, {}
    for v in per.values():
        for c, x in v.items():
            sums[c] = sums.get(c, 0.0) + x
            cnt[c] = cnt.get(c, 0) + 1
    m = {c: sums[c] / cnt[c] for c in sums}
    cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / 8

    def frac(num, den):
        return f"{num / den:.3g}" if den else "-"

    parts = [label, f"{cyc:.4g}" if cyc else "-"]
    parts.append(frac(m.get("TA_TA_BUSY_sum", 0.0), 256 * cyc) if "TA_TA_BUSY_sum" in m else "-")
    parts.append(frac(m.get("TA_ADDR_STALLED_BY_TC_CYCLES_sum", 0.0), m.get("TA_TA_BUSY_sum", 0.0))
                 if "TA_ADDR_STALLED_BY_TC_CYCLES_sum" in m else "-")
    if "TCC_EA0_RDREQ_sum" in m:
        parts.append(f"{m['TCC_EA0_RDREQ_LEVEL_sum'] / m['TCC_EA0_RDREQ_sum']:.0f}")
        parts.append(f"{m['TCC_EA0_RDREQ_LEVEL_sum'] / cyc:.3g}" if cyc else "-")
        parts.append(frac(m.get("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", 0.0), 128 * cyc))
        parts.append(frac(m.get("TCC_BUSY_sum", 0.0), 128 * cyc))
    else:
        parts += ["-"] * 4
    parts.append(frac(m.get("TCP_PENDING_STALL_CYCLES_sum", 0.0), 256 * cyc) if "TCP_PENDING_STALL_CYCLES_sum" in m else "-")
    if "SQ_WAVE_CYCLES" in m:
        w = m["SQ_WAVE_CYCLES"]
        parts.append(f"{m['SQ_WAIT_ANY'] / w:.2f} / {m['SQ_WAIT_INST_ANY'] / w:.2f} / {m['SQ_ACTIVE_INST_ANY'] / w:.2f}")
    else:
        parts.append("-")
    print("| " + " | ".join(parts) + " |")


# ---- power and clock while a workload runs -----------------------------------

def _under_profiler() -> bool:
    """True when this process runs under rocprofv3, which sets these for the
    program it profiles: amd-smi is not started then (a child process of a
    profiled program would start with the profiler's library preloaded)."""
    return "ROCPROFILER_LIBRARY_CTOR" in os.environ or "ROCPROF_OUTPUT_PATH" in os.environ


def _smi_sample():
    """Socket power (W) and the mean of the 8 XCDs' gfx clocks (MHz), from one
    `amd-smi metric -p -c` reading of GPU 0, run as a child process; (None,
    None) if unavailable or under a profiler."""
    import re
    import subprocess

    if _under_profiler():
        return None, None
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True, text=True,
                             timeout=10).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None, None
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
    clks = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", out)]
    return (float(pw.group(1)) if pw else None), (sum(clks) / len(clks) if clks else None)


def observed_clock(run, ms_per_call, seconds=2.5, warm_s=0.5):
    """Mean gfx clock (MHz) and socket power (W) of GPU 0 sampled with
    amd-smi while `run` goes back to back for about `seconds`, after the timed
    region and `warm_s` of unsampled calls (the board ramps up again after the
    idle host work before it); None where amd-smi gives nothing."""
    import threading

    if _under_profiler():
        return {"gfx_clock_mhz": None, "socket_power_w": None, "samples": 0,
                "tool": "not sampled: running under a profiler"}
    per = max(ms_per_call, 1e-3)
    _time_region(run, max(1, int(warm_s * 1e3 / per)), 0)
    calls = max(1, int(seconds * 1e3 / per))
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append(_smi_sample())
            stop.wait(0.2)

    th = threading.Thread(target=sampler)
    th.start()
    _time_region(run, calls, 0)
    stop.set()
    th.join()
    pw = [p for p, _ in samples if p is not None]
    ck = [c for _, c in samples if c is not None]
    return {"gfx_clock_mhz": round(sum(ck) / len(ck), 1) if ck else None,
            "socket_power_w": round(sum(pw) / len(pw), 1) if pw else None,
            "samples": len(samples), "tool": "amd-smi metric -p -c, after the timed region and 0.5 s of warm calls"}


def sweep(steps=10, warmup=3):
    """Rates over shapes beyond the named workloads (no oracle check): prefill
    bf16 at d = 128 over sequence lengths (MHA, B * S = 32768 tokens, causal and
    not; GQA 32/8 up to S = 65536), d = 64, fp16 and fp8; the backward; int8-KV
    decode over cache lengths (B = 64, GQA 32/8, 2048-token splits, at most 64), and once with a
    cache length that leaves the scale rows unaligned (2-byte scale loads).
    Prints one markdown row per shape."""
    import torch

    F = fa_inputs.FwdConfig
    rows = []
    for causal in (True, False):
        for S in (512, 1024, 2048, 4096, 8192, 16384, 32768):
            B = max(1, 32768 // S)
            rows.append(F(f"bf16 MHA", "bf16", B, 16, 16, S, S, 128, causal))
    for S in (4096, 16384, 65536):
        rows.append(F("bf16 GQA 32/8", "bf16", 1, 32, 8, S, S, 128, True))
    for S in (512, 1024, 2048, 8192):
        rows.append(F("bf16 MHA d=64", "bf16", 32768 // S, 16, 16, S, S, 64, True))
    rows.append(F("fp16 MHA", "f16", 16, 16, 16, 2048, 2048, 128, True))
    for S, causal in ((1024, False), (4096, False), (16384, False), (4096, True)):
        rows.append(F("fp8 MHA", "fp8", max(1, 32768 // S), 16, 16, S, S, 128, causal, out_dtype="bf16"))
    for S in (2048, 8192, 16384):
        rows.append(fa_inputs.BwdConfig("backward bf16 GQA 32/8", "bf16", max(1, 16384 // S), 32, 8, S, S, 128,
                                        True))
    for L in (4096, 16384, 32768, 131072):
        rows.append(fa_inputs.DecodeConfig("decode int8 GQA 32/8", 64, 32, 8, L, 128, min(64, max(1, L // 2048))))
    # a cache length that is not a multiple of 8: scale rows not 16-byte aligned, 2-byte scale loads
    rows.append(fa_inputs.DecodeConfig("decode int8 GQA 32/8, unaligned scale rows", 64, 32, 8, 32764, 128, 16))
    print("| kind | B | Hq/Hkv | S or L | d | causal | ms per call | rate | fraction of peak |")
    print("|---|---|---|---|---|---|---|---|---|")
    for cfg in rows:
        r = _runner(cfg)
        ms, _ = _time_region(r.run, steps, warmup)
        work, unit = work_and_unit(cfg)
        if unit == "GB/s":
            rate = work / (ms * 1e-3) / 1e9
            frac = f"{rate / PEAK_HBM_GBS:.1%} HBM"
            shape = (cfg.B, f"{cfg.Hq}/{cfg.Hkv}", cfg.L, cfg.d, "-")
        else:
            rate = work / (ms * 1e-3) / 1e12
            peak = {"f32": PEAK_F32_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(cfg.dtype, PEAK_BF16_TFLOPS)
            frac = f"{rate / peak:.1%} of its dtype's peak"
            if cfg.dtype == "fp8":
                frac += f", {rate / PEAK_BF16_TFLOPS:.1%} of bf16"
            shape = (cfg.B, f"{cfg.Hq}/{cfg.Hkv}", cfg.Sq, cfg.d, "yes" if cfg.causal else "no")
        print(f"| {cfg.name} | " + " | ".join(str(x) for x in shape) + f" | {ms:.4f} | {rate:.1f} {unit} | {frac} |",
              flush=True)
        del r
        torch.cuda.empty_cache()


def power_study(names, seconds=4.0):
    """For each workload (and the vendor bf16 GEMM, torch.matmul of 8192^3,
    as a reference for a plain contraction on this part): run it back to back
    for `seconds` while sampling socket power and gfx clocks; prints one
    markdown row each: achieved rate, mean and peak power, mean clock."""
    import threading

    import torch

    print("| workload | rate | mean socket power W | peak W | mean gfx clock MHz | samples |")
    print("|---|---|---|---|---|---|")
    # the GEMM first: it also brings the board to its steady power and temperature
    jobs = [("vendor bf16 GEMM 8192^3 (torch.matmul)", "gemm")] + [(n, None) for n in names]
    for name, kind in jobs:
        if kind == "gemm":
            a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
            b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
            c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
            run = lambda: torch.matmul(a, b, out=c)  # noqa: E731
            work, unit = 2 * 8192 ** 3, "TFLOP/s"
        else:
            cfg = workload(name)
            run = _runner(cfg).run
            work, unit = work_and_unit(cfg)
        ms, _ = _time_region(run, 10, 5)  # warm, and per-call time for the loop length
        calls = max(1, int(seconds * 1e3 / ms))
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                samples.append(_smi_sample())
                stop.wait(0.2)

        th = threading.Thread(target=sampler)
        th.start()
        ms, _ = _time_region(run, calls, 0)
        stop.set()
        th.join()
        pw = [p for p, _ in samples if p is not None]
        ck = [c for _, c in samples if c is not None]
        rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        print(f"| {name} | {rate:.1f} {unit} | {sum(pw) / max(1, len(pw)):.0f} | {max(pw, default=0):.0f} | "
              f"{sum(ck) / max(1, len(ck)):.0f} | {len(samples)} |", flush=True)
        del run
        torch.cuda.empty_cache()


# ---- main ---------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default="all", help="other workloads to time: all, none or a comma list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-pmc", action="store_true",
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs into profiles/hbm_traffic.json")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30)
    ap.add_argument("--calib-kernel", default="MulFunctor")
    ap.add_argument("--kernel", default="fwd_mfma16_kernel")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="summarise a rocprofv3 kernel trace of this script against --bench-json")
    ap.add_argument("--bench-json")
    ap.add_argument("--summarize-counters", metavar="DIRS",
                    help="summarise rocprofv3 --pmc runs (comma-separated dirs) of --workload for --kernel")
    ap.add_argument("--summarize-memory", metavar="DIRS",
                    help="summarise memory-pipeline rocprofv3 --pmc runs (comma-separated dirs) of --kernel")
    ap.add_argument("--label", default="")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="time vendor read-only and copy kernels over the decode workload's byte count")
    ap.add_argument("--sweep", action="store_true",
                    help="rates over sequence lengths, head dims, dtypes and cache lengths (markdown rows)")
    ap.add_argument("--power-study", metavar="NAMES",
                    help="sample socket power and clocks while each listed workload (comma list) runs, "
                         "and the vendor bf16 GEMM")
    a = ap.parse_args()
    if a.summarize_memory:
        summarize_memory(a.summarize_memory, a.kernel, a.label or a.kernel)
        return
    if a.stream_ceiling:
        import torch

        torch.cuda.set_device(0)
        stream_ceiling()
        return
    if a.sweep:
        import torch

        import tiled_exact_attention_fa_amd as fa

        fa.load()
        torch.cuda.set_device(0)
        sweep()
        return
    if a.power_study:
        import torch

        import tiled_exact_attention_fa_amd as fa

        fa.load()
        torch.cuda.set_device(0)
        power_study([n for n in a.power_study.split(",") if n])
        return
    if a.summarize_counters:
        summarize_counters(a.summarize_counters, a.kernel, a.workload)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace, a.bench_json)
        return
    if a.summarize_pmc:
        summarize_pmc(a)
        return
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the path runs on a single device and has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_exact_attention_fa_amd as fa

    fa.load()
    torch.cuda.set_device(0)
    cpu_on = not a.no_cpu_baseline
    head = measure(a.workload, a.steps, a.warmup, check_budget=12.0 if cpu_on else 0.0, clock=True)
    cfg = workload(a.workload)

    extras = {}
    names = [n for n in list(fa_inputs.CONFIGS) + list(fa_inputs.BWD_CONFIGS) + list(fa_inputs.KV_CONFIGS)
             + list(fa_inputs.FP8_VARIANT_CONFIGS) + list(fa_inputs.SOFT_EXP2_CONFIGS)
             + list(fa_inputs.NO_LSE_CONFIGS) + list(fa_inputs.BWD_VARIANT_CONFIGS) if n != a.workload]
    if a.extra == "none":
        names = []
    elif a.extra != "all":
        names = [n for n in a.extra.split(",") if n]
    for n in names:
        # the five configurations also get the oracle baseline and error check
        budget = 4.0 if cpu_on and n in fa_inputs.CONFIGS else 0.0
        try:
            extras[n] = measure(n, max(3, a.steps // 5), max(2, a.warmup // 2), check_budget=budget)
        except Exception as e:  # an unbuilt kernel is reported, not hidden
            extras[n] = {"error": f"{type(e).__name__}: {e}"}
        print(f"# {n}: {json.dumps(extras[n])}", file=sys.stderr, flush=True)

    cpu = None
    if "cpu_baseline" in head:
        # in the metric's own unit (TFLOP/s or GB/s)
        cpu = dict(head["cpu_baseline"])
        if cpu["unit"] == "GFLOP/s":
            cpu["value"], cpu["unit"] = cpu["value"] / 1e3, "TFLOP/s"

    dtype = {"f32": "f32", "bf16": "bf16", "f16": "f16", "fp8": "fp8_e4m3"}.get(getattr(cfg, "dtype", ""), "bf16")
    conf = {"workload": a.workload}
    if isinstance(cfg, fa_inputs.FwdConfig):
        conf.update({"B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "seq_len": cfg.Sq, "d": cfg.d,
                     "causal": cfg.causal, "lse": cfg.lse})
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": conf,
        "ms_median": head["ms_median"],
        "ms_min": head["ms_min"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "max_abs_err": head.get("max_abs_err"),
        "observed": head.get("observed"),
        "workloads": extras,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
