"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds no attention arithmetic: only random draws, dtype casts and the input-side
quantisers that turn float draws into the low-precision operands (fp8 e4m3
tensors with a per-tensor scale, an int8 KV cache with per-token-per-head fp16
scales).  The GPU library never imports it.

Recipe (the same on every device; ``device`` only chooses where the generator
runs, so CPU and GPU draws differ but each is deterministic for a given seed):

* a torch.Generator on ``device`` seeded with ``seed`` draws float32 N(0,1) in the
  order Q, K, V (BHSD shapes), then the outlier row indices; casts to bf16/fp16
  round to nearest even;
* long-context outlier keys: per (batch, kv head), exactly round(0.01 * Sk)
  distinct key rows picked by a seeded permutation are multiplied by 8 in float32
  before the cast (a power-of-two factor, so the multiply is exact);
* fp8: per-tensor scale s = float32(absmax / 448); codes = E4M3FN(x / s), round to
  nearest even, clamped to +-448 before the cast;
* int8 KV cache: per (batch, kv head, token) scale sc = fp16(absmax_over_d / 127);
  code = clamp(rint(x / float(sc)), -127, 127), 0 where sc == 0.  The decode cache
  is drawn one batch entry at a time (seed (seed << 20) + b, K then V) so that no
  full-size float32 temporary is needed; the query uses seed (seed << 20) + B.
* fp8 KV cache: the same draws, with sc = fp16(absmax_over_d / 448) and
  code = E4M3FN(clamp(x / float(sc), +-448)), round to nearest even;
* residual window: bf16 N(0,1) keys then values [B, Hkv, W, d] drawn with seed
  (seed << 20) + B + 1, every sequence attending all W of them unless the config
  lists window lengths;
* append: new key rows then value rows [B, H, T, d] bf16 N(0,1) from seed
  (seed << 20) + 7, written at each sequence's position pos0;
* backward: the forward's inputs, then dO [B, Hq, Sq, d] N(0,1) from seed
  (seed << 20) + 5, cast like the inputs;
* fp8 block-scaled prefill and its quantiser: the bf16 draws of the forward
  recipe (the library's own quantiser turns them into codes); the rotation's
  +-1 signs [d] are drawn from seed (seed << 20) + 9, uniform [0, 1) < 0.5
  giving -1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0
INT8_QMAX = 127


@dataclass(frozen=True)
class FwdConfig:
    name: str
    dtype: str  # "f32" | "bf16" | "f16" | "fp8"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    causal: bool
    outlier_frac: float = 0.0
    out_dtype: str = ""
    lse: bool = True  # whether the call asks for the LSE output

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    num_splits: int
    seq_lens: tuple = field(default=())
    kv_format: str = "int8"  # "int8" | "fp8"
    W: int = 0  # residual window capacity (0: none)
    recent_lens: tuple = field(default=())

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class BwdConfig(FwdConfig):
    """A backward workload: the forward's inputs plus a dO drawn after them."""


@dataclass(frozen=True)
class AppendConfig:
    name: str
    B: int
    H: int
    T: int
    L: int
    d: int
    kv_format: str  # "int8" | "fp8"
    pos0: int = 0


@dataclass(frozen=True)
class Fp8BlockConfig(FwdConfig):
    """fp8 prefill on codes with 64-row block scales (Q and K rotated when
    ``rotate``), quantised from the bf16 draws of the same shape."""
    rotate: bool = False


@dataclass(frozen=True)
class QuantConfig:
    """The block quantiser over Q, K and V of one prefill (Q and K rotated when
    ``rotate``)."""
    name: str
    B: int
    H: int
    S: int
    d: int
    rotate: bool


# The five workloads: a tiny fp32 case, causal bf16 prefill, long-context GQA
# prefill with outlier keys, fp8 prefill and int8-KV split decode.
CONFIGS = {
    "fp32_s128_d64": FwdConfig("fp32_s128_d64", "f32", 1, 1, 1, 128, 128, 64, False),
    "bf16_b4_h16_s2048_causal": FwdConfig("bf16_b4_h16_s2048_causal", "bf16", 4, 16, 16, 2048, 2048, 128, True),
    "bf16_gqa32x8_s16384_causal_outlier": FwdConfig(
        "bf16_gqa32x8_s16384_causal_outlier", "bf16", 1, 32, 8, 16384, 16384, 128, True, outlier_frac=0.01),
    "fp8_b8_h16_s4096": FwdConfig("fp8_b8_h16_s4096", "fp8", 8, 16, 16, 4096, 4096, 128, False, out_dtype="bf16"),
    "decode_int8_b64_gqa32x8_L32768": DecodeConfig("decode_int8_b64_gqa32x8_L32768", 64, 32, 8, 32768, 128, 16),
}

# The backward of the two causal bf16 prefill workloads (same inputs, plus a
# N(0,1) gradient dO of the output).
BWD_CONFIGS = {
    "bwd_bf16_b4_h16_s2048_causal": BwdConfig("bwd_bf16_b4_h16_s2048_causal", "bf16", 4, 16, 16, 2048, 2048, 128, True),
    "bwd_bf16_gqa32x8_s16384_causal_outlier": BwdConfig(
        "bwd_bf16_gqa32x8_s16384_causal_outlier", "bf16", 1, 32, 8, 16384, 16384, 128, True, outlier_frac=0.01),
}

# The cache's other formats and its write side, at the decode workload's sizes:
# the same decode over an fp8 cache, the int8 decode with a 128-token bf16
# residual window, and the quantise-on-append of a 4096-token chunk for all 64
# sequences (positions 28672 .. 32767 of the 32768-slot cache).
KV_CONFIGS = {
    "decode_fp8_b64_gqa32x8_L32768": DecodeConfig("decode_fp8_b64_gqa32x8_L32768", 64, 32, 8, 32768, 128, 16,
                                                  kv_format="fp8"),
    "decode_int8_window128_b64_gqa32x8_L32768": DecodeConfig(
        "decode_int8_window128_b64_gqa32x8_L32768", 64, 32, 8, 32768, 128, 16, W=128),
    "append_int8_b64_h8_t4096": AppendConfig("append_int8_b64_h8_t4096", 64, 8, 4096, 32768, 128, "int8", 28672),
    "append_fp8_b64_h8_t4096": AppendConfig("append_fp8_b64_h8_t4096", 64, 8, 4096, 32768, 128, "fp8", 28672),
}

@dataclass(frozen=True)
class Fp8PBf16Config(FwdConfig):
    """An fp8 prefill workload run with the probabilities rounded to bf16 for
    P V (fa_fwd_params.fp8_p_bf16 = 1); same inputs as FwdConfig."""


@dataclass(frozen=True)
class SoftExp2Config(FwdConfig):
    """A bf16/fp16 prefill workload run with a quarter of the exponentials in
    software (fa_fwd_params.soft_exp2 = 1); same inputs as FwdConfig."""


# The long-context workload with the software-exponential split.
SOFT_EXP2_CONFIGS = {
    "softexp2_bf16_gqa32x8_s16384_causal_outlier": SoftExp2Config(
        "softexp2_bf16_gqa32x8_s16384_causal_outlier", "bf16", 1, 32, 8, 16384, 16384, 128, True, outlier_frac=0.01),
}

@dataclass(frozen=True)
class PingPongBwdConfig(BwdConfig):
    """A backward workload run with the dK/dV kernel's two-role wave schedule
    (fa_bwd_params.wave_pingpong = 1); same inputs as BwdConfig."""


# The long-context backward with the two-role schedule.
BWD_VARIANT_CONFIGS = {
    "bwd_pingpong_bf16_gqa32x8_s16384_causal_outlier": PingPongBwdConfig(
        "bwd_pingpong_bf16_gqa32x8_s16384_causal_outlier", "bf16", 1, 32, 8, 16384, 16384, 128, True,
        outlier_frac=0.01),
}

# The long-context workload called without an LSE output (the workload as
# specified names only O; the kernel then skips the unrounded row sum).
NO_LSE_CONFIGS = {
    "nolse_bf16_gqa32x8_s16384_causal_outlier": FwdConfig(
        "nolse_bf16_gqa32x8_s16384_causal_outlier", "bf16", 1, 32, 8, 16384, 16384, 128, True, outlier_frac=0.01,
        lse=False),
}

# The fp8 accuracy variants at the fp8 workload's shape: the forward on
# block-scaled codes, the quantiser that makes them, and the per-tensor fp8
# workload with bf16 probabilities.
FP8_VARIANT_CONFIGS = {
    "fp8_pbf16_b8_h16_s4096": Fp8PBf16Config("fp8_pbf16_b8_h16_s4096", "fp8", 8, 16, 16, 4096, 4096, 128, False,
                                             out_dtype="bf16"),
    "fp8_block_rot_b8_h16_s4096": Fp8BlockConfig("fp8_block_rot_b8_h16_s4096", "fp8", 8, 16, 16, 4096, 4096, 128,
                                                 False, out_dtype="bf16", rotate=True),
    "fp8_quant_rot_b8_h16_s4096": QuantConfig("fp8_quant_rot_b8_h16_s4096", 8, 16, 4096, 128, True),
}

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def quantize_fp8_per_tensor(x: torch.Tensor):
    """float tensor -> (E4M3FN codes as torch.float8_e4m3fn, float32 scale).

    s = absmax / 448 in float32; codes = RNE(x / s) clamped to +-448."""
    xf = x.float()
    amax = xf.abs().max()
    s = (amax / E4M3_MAX).to(torch.float32)
    if float(s) == 0.0:
        s = torch.tensor(1.0, dtype=torch.float32, device=x.device)
    y = (xf / s).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), float(s)


def quantize_int8_tokhead(x: torch.Tensor):
    """float tensor [..., T, d] -> (int8 codes [..., T, d], fp16 scales [..., T]).

    Symmetric per-token scale sc = fp16(absmax_d / 127); code = clamp(rint(x/sc))."""
    xf = x.float()
    amax = xf.abs().amax(dim=-1)
    sc = (amax / INT8_QMAX).to(torch.float16)
    scf = sc.float()
    safe = torch.where(scf > 0, scf, torch.ones_like(scf))
    qv = torch.round(xf / safe[..., None]).clamp_(-INT8_QMAX, INT8_QMAX)
    qv = torch.where(scf[..., None] > 0, qv, torch.zeros_like(qv))
    return qv.to(torch.int8), sc


def quantize_fp8_tokhead(x: torch.Tensor):
    """float tensor [..., T, d] -> (E4M3FN codes [..., T, d] as uint8, fp16 scales [..., T]).

    Symmetric per-token scale sc = fp16(absmax_d / 448); code = E4M3FN(x / sc)
    after clamping to +-448, round to nearest even."""
    xf = x.float()
    amax = xf.abs().amax(dim=-1)
    sc = (amax / E4M3_MAX).to(torch.float16)
    scf = sc.float()
    safe = torch.where(scf > 0, scf, torch.ones_like(scf))
    y = (xf / safe[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    codes = torch.where(scf[..., None] > 0, codes, torch.zeros_like(codes))
    return codes, sc


def make_fwd_inputs(cfg: FwdConfig, seed: int = 0, device="cpu"):
    """Returns a dict with q, k, v (in the config's input dtype) and, for fp8,
    the float32 per-tensor scales q_scale, k_scale, v_scale."""
    g = _gen(device, seed)
    qf = torch.randn(cfg.B, cfg.Hq, cfg.Sq, cfg.d, generator=g, device=device, dtype=torch.float32)
    kf = torch.randn(cfg.B, cfg.Hkv, cfg.Sk, cfg.d, generator=g, device=device, dtype=torch.float32)
    vf = torch.randn(cfg.B, cfg.Hkv, cfg.Sk, cfg.d, generator=g, device=device, dtype=torch.float32)
    if cfg.outlier_frac > 0:
        n_out = int(round(cfg.outlier_frac * cfg.Sk))
        for b in range(cfg.B):
            for h in range(cfg.Hkv):
                idx = torch.randperm(cfg.Sk, generator=g, device=device)[:n_out]
                kf[b, h, idx] *= 8.0
    if cfg.dtype == "fp8":
        q8, qs = quantize_fp8_per_tensor(qf)
        k8, ks = quantize_fp8_per_tensor(kf)
        v8, vs = quantize_fp8_per_tensor(vf)
        return {"q": q8, "k": k8, "v": v8, "q_scale": qs, "k_scale": ks, "v_scale": vs}
    dt = _TORCH_DT[cfg.dtype]
    return {"q": qf.to(dt), "k": kf.to(dt), "v": vf.to(dt)}


def make_bwd_inputs(cfg: BwdConfig, seed: int = 0, device="cpu"):
    """The forward inputs of the same seed plus dout [B,Hq,Sq,d] in the input
    dtype, drawn N(0,1) from seed (seed << 20) + 5."""
    x = make_fwd_inputs(cfg, seed=seed, device=device)
    g = _gen(device, (seed << 20) + 5)
    dout = torch.randn(cfg.B, cfg.Hq, cfg.Sq, cfg.d, generator=g, device=device, dtype=torch.float32)
    x["dout"] = dout.to(_TORCH_DT[cfg.dtype])
    return x


def make_decode_inputs(cfg: DecodeConfig, seed: int = 0, device="cpu"):
    """Returns q [B,Hq,d] bf16, k/v codes [B,Hkv,L,d] (int8, or uint8 E4M3FN
    bytes for the fp8 format), k/v scales [B,Hkv,L] fp16 and seq_lens [B] int32
    (all L unless the config lists lengths); with a window also k_recent /
    v_recent [B,Hkv,W,d] bf16 and recent_lens [B] int32."""
    B, Hkv, L, d = cfg.B, cfg.Hkv, cfg.L, cfg.d
    quant = quantize_int8_tokhead if cfg.kv_format == "int8" else quantize_fp8_tokhead
    cdt = torch.int8 if cfg.kv_format == "int8" else torch.uint8
    kc = torch.empty(B, Hkv, L, d, dtype=cdt, device=device)
    vc = torch.empty(B, Hkv, L, d, dtype=cdt, device=device)
    ks = torch.empty(B, Hkv, L, dtype=torch.float16, device=device)
    vs = torch.empty(B, Hkv, L, dtype=torch.float16, device=device)
    for b in range(B):
        g = _gen(device, (seed << 20) + b)
        kf = torch.randn(Hkv, L, d, generator=g, device=device, dtype=torch.float32)
        kc[b], ks[b] = quant(kf)
        del kf
        vf = torch.randn(Hkv, L, d, generator=g, device=device, dtype=torch.float32)
        vc[b], vs[b] = quant(vf)
        del vf
    g = _gen(device, (seed << 20) + B)
    q = torch.randn(B, cfg.Hq, d, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    if cfg.seq_lens:
        lens = torch.tensor(cfg.seq_lens, dtype=torch.int32, device=device)
    else:
        lens = torch.full((B,), L, dtype=torch.int32, device=device)
    out = {"q": q, "k": kc, "v": vc, "k_scale": ks, "v_scale": vs, "seq_lens": lens}
    if cfg.W > 0:
        g = _gen(device, (seed << 20) + B + 1)
        out["k_recent"] = torch.randn(B, Hkv, cfg.W, d, generator=g, device=device).to(torch.bfloat16)
        out["v_recent"] = torch.randn(B, Hkv, cfg.W, d, generator=g, device=device).to(torch.bfloat16)
        rl = cfg.recent_lens if cfg.recent_lens else (cfg.W,) * B
        out["recent_lens"] = torch.tensor(rl, dtype=torch.int32, device=device)
    return out


def make_append_inputs(cfg: AppendConfig, seed: int = 0, device="cpu"):
    """Returns new rows k_new / v_new [B,H,T,d] bf16, empty caches [B,H,L,d]
    (int8, or uint8 E4M3FN bytes) with fp16 scales [B,H,L], and positions [B]
    int32 (all pos0)."""
    g = _gen(device, (seed << 20) + 7)
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    kn = torch.randn(*shape, generator=g, device=device).to(torch.bfloat16)
    vn = torch.randn(*shape, generator=g, device=device).to(torch.bfloat16)
    cdt = torch.int8 if cfg.kv_format == "int8" else torch.uint8
    kc = torch.zeros(cfg.B, cfg.H, cfg.L, cfg.d, dtype=cdt, device=device)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(cfg.B, cfg.H, cfg.L, dtype=torch.float16, device=device)
    vs = torch.zeros_like(ks)
    pos = torch.full((cfg.B,), cfg.pos0, dtype=torch.int32, device=device)
    return {"k_new": kn, "v_new": vn, "k_cache": kc, "v_cache": vc, "k_scale": ks, "v_scale": vs,
            "positions": pos}


def make_rotation_signs(d: int, seed: int = 0, device="cpu"):
    """+-1 float32 signs [d] of the random-sign Hadamard rotation."""
    g = _gen(device, (seed << 20) + 9)
    u = torch.rand(d, generator=g, device=device)
    return torch.where(u < 0.5, -1.0, 1.0).to(torch.float32)


def make_quant_inputs(cfg: QuantConfig, seed: int = 0, device="cpu"):
    """bf16 q, k, v [B, H, S, d] of the forward recipe and the rotation signs."""
    fc = FwdConfig(cfg.name, "bf16", cfg.B, cfg.H, cfg.H, cfg.S, cfg.S, cfg.d, False)
    x = make_fwd_inputs(fc, seed=seed, device=device)
    x["signs"] = make_rotation_signs(cfg.d, seed, device) if cfg.rotate else None
    return x
