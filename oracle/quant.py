"""Quantisers of the KV-cache write side and of fp8 prefill inputs — TEST INFRASTRUCTURE ONLY (see package doc).

KV-cache quantisation overview, section 3 ("where quantisation can sit"): before
a key or value row enters the cache it is turned from FP16/BF16 into a low-bit
code plus the metadata needed to read it back (a scale); FP8 and INT8 are two of
the storage forms the section lists, and the read side maps code x scale back
into the compute domain.  The overview does not fix the granularity or the
rounding; the readings taken here are:

* symmetric codes, no zero point; one fp16 scale per (batch, cache head, token);
* sc = fp16(fp32(absmax / QMAX)) with QMAX = 127 (int8) or 448 (E4M3FN, the
  largest finite value of the format), the fp32 quotient clamped to 65504 first
  so that the scale never becomes infinite; round to nearest even at each step;
* sc == 0 (an all-zero row, or a row so small that its scale underflows fp16)
  stores code 0 everywhere;
* otherwise y = fp32(x) / fp32(sc), one correctly rounded fp32 division — the
  precision in which the integer code is decided, on both sides of a parity test;
* int8: code = clamp(rint(y), -127, 127), rint rounding half to even;
* fp8:  code = the E4M3FN byte nearest to clamp(y, -448, 448), ties to the even
  mantissa; the sign of y is kept, so a negative y that rounds to zero gives 0x80.

The E4M3FN encoder is written from the format's definition (1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, subnormals m/8 x 2^-6, largest
finite 448, no infinities); it shares nothing with the GPU path.
"""

from __future__ import annotations

import math

import numpy as np

INT8_QMAX = 127.0
E4M3_QMAX = 448.0
F16_MAX = 65504.0


def _f32(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x.astype(np.float32)
    import torch

    return x.detach().to("cpu", torch.float32).numpy()


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN byte to each float64 value, ties to even mantissa,
    saturating at +-448.  Returns uint8 codes of the same shape."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_QMAX)
    # binade exponent, held inside the normal range; below 2^-6 the spacing is
    # that of the subnormals, 2^-9
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    spacing = np.exp2(e - 3)
    val = np.rint(a / spacing) * spacing  # a / spacing is exact (power of two)
    val = np.minimum(val, E4M3_QMAX)
    normal = val >= 2.0 ** -6
    with np.errstate(divide="ignore"):
        en = np.floor(np.log2(np.where(normal, val, 1.0)))
    efield = np.where(normal, en + 7, 0)
    mfield = np.where(normal, val / np.exp2(en) * 8 - 8, val / 2.0 ** -9)
    code = (neg.astype(np.int64) << 7) | (efield.astype(np.int64) << 3) | mfield.astype(np.int64)
    return code.astype(np.uint8)


def quantize_kv_tokhead(x, fmt: str):
    """Rows x [..., T, d] (bf16/fp16 values, numpy or torch) -> (codes, scales).

    fmt "int8": codes int8; fmt "fp8": codes uint8 E4M3FN bytes.  scales are
    float16 [..., T].  Every step follows the readings in the module doc."""
    if fmt not in ("int8", "fp8"):
        raise ValueError(fmt)
    xf = _f32(x)
    qmax = np.float32(INT8_QMAX if fmt == "int8" else E4M3_QMAX)
    amax = np.max(np.abs(xf), axis=-1) if xf.shape[-1] else np.zeros(xf.shape[:-1], np.float32)
    sc32 = np.minimum(amax.astype(np.float32) / qmax, np.float32(F16_MAX))
    sc = sc32.astype(np.float16)
    scf = sc.astype(np.float32)
    live = scf > 0
    y = xf / np.where(live, scf, np.float32(1.0))[..., None]  # float32 / float32
    if fmt == "int8":
        codes = np.clip(np.rint(y), -INT8_QMAX, INT8_QMAX)
        codes = np.where(live[..., None], codes, 0).astype(np.int8)
    else:
        codes = e4m3_encode(np.clip(y.astype(np.float64), -E4M3_QMAX, E4M3_QMAX))
        codes = np.where(live[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, sc


def kv_append_ref(cache_codes, cache_scales, rows, positions, fmt: str):
    """Writes quantised rows into copies of a cache.

    cache_codes [B, H, L, d], cache_scales [B, H, L]; rows [B, H, T, d];
    positions [B] (first cache slot written for batch b; None = 0).  Row t of
    batch b goes to slot positions[b] + t; rows whose slot falls outside
    [0, L) are dropped.  Returns the new (codes, scales)."""
    codes = np.array(cache_codes, copy=True)
    scales = np.array(cache_scales, copy=True)
    qc, qs = quantize_kv_tokhead(rows, fmt)
    B, H, T = qc.shape[:3]
    L = codes.shape[2]
    pos = [0] * B if positions is None else [int(p) for p in np.asarray(positions).tolist()]
    for b in range(B):
        for t in range(T):
            s = pos[b] + t
            if 0 <= s < L:
                codes[b, :, s] = qc[b, :, t]
                scales[b, :, s] = qs[b, :, t]
    return codes, scales


# ---- fp8 inputs of the prefill: block scales and incoherent processing ----
#
# FlashAttention-3 page, producer/consumer pseudocode box ("FP8 path") and the
# closing answer: fp8 attention keeps its accuracy with block-wise
# quantisation of Q, K and V and with incoherent processing (the page gives no
# formulas).  Readings taken here:
#   * a block is 64 consecutive rows (tokens) of one (batch, head) slice, with
#     one fp32 scale s, the smallest power of two at or above fp32(absmax / 448)
#     (shared power-of-two block exponents, as the OCP microscaling formats
#     use); s == 0 stores code 0 everywhere; code = E4M3FN(clamp(y / s, +-448)),
#     nearest even (y / s is exact).  A power of two keeps every ratio of two
#     block scales a power of two, so an attention kernel can fold a V block's
#     scale into the probabilities before their own e4m3 rounding without
#     adding a rounding step;
#   * incoherent processing multiplies each row of Q and of K by the same
#     orthogonal matrix R = diag(signs) H / sqrt(d) (H the Sylvester-Hadamard
#     matrix, signs a random +-1 vector) before quantising: (Q R)(K R)^T =
#     Q K^T exactly, while an outlier channel is spread over all d channels.
#     It is evaluated in float32 as the iterative fast transform — stages
#     h = 1, 2, 4, ..., d/2, each mapping the pair (a at i, b at i + h) of an
#     aligned block of 2h to (a + b, a - b) — followed by one multiply by
#     fp32(1 / sqrt(d)), the order in which the codes are decided.

FP8_BLOCK_ROWS = 64


def pow2_at_or_above(v) -> np.ndarray:
    """Smallest power of two >= v for float32 v > 0 (0 stays 0), in float32."""
    v = np.asarray(v, dtype=np.float32)
    m, e = np.frexp(v)  # v = m 2^e, m in [0.5, 1)
    p = np.where(m == 0.5, np.ldexp(np.float32(1.0), e - 1), np.ldexp(np.float32(1.0), e))
    return np.where(v > 0, p, np.float32(0.0)).astype(np.float32)


def hadamard_rotate_fp32(x, signs) -> np.ndarray:
    """Rows x [..., d] (float32 values) times diag(signs) H / sqrt(d), in float32,
    by the stage order stated above.  d must be a power of two."""
    y = np.array(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(*y.shape[:-1], d)
        h *= 2
    return y * np.float32(1.0 / math.sqrt(d))


def quantize_fp8_blocks(x, signs=None, block_rows: int = FP8_BLOCK_ROWS):
    """x [B, H, S, d] (bf16/fp16/fp32 values) -> (codes uint8 [B, H, S, d],
    scales float32 [B, H, ceil(S / block_rows)]), optionally rotated first."""
    xf = _f32(x)
    if signs is not None:
        xf = hadamard_rotate_fp32(xf, signs)
    B, H, S, d = xf.shape
    nb = (S + block_rows - 1) // block_rows
    codes = np.zeros((B, H, S, d), dtype=np.uint8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for blk in range(nb):
        r0, r1 = blk * block_rows, min(S, (blk + 1) * block_rows)
        part = xf[:, :, r0:r1]
        amax = np.max(np.abs(part), axis=(2, 3)) if r1 > r0 else np.zeros((B, H), np.float32)
        s = pow2_at_or_above((amax.astype(np.float32) / np.float32(E4M3_QMAX)).astype(np.float32))
        scales[:, :, blk] = s
        live = s > 0
        y = part / np.where(live, s, np.float32(1.0))[:, :, None, None]
        c = e4m3_encode(np.clip(y.astype(np.float64), -E4M3_QMAX, E4M3_QMAX))
        codes[:, :, r0:r1] = np.where(live[:, :, None, None], c, np.uint8(0))
    return codes, scales


def dequant_fp8_blocks_fp64(codes, scales, block_rows: int = FP8_BLOCK_ROWS) -> np.ndarray:
    """codes [B, H, S, d] E4M3FN bytes, scales [B, H, nblk] -> float64 values."""
    from .e4m3 import e4m3_decode

    S = codes.shape[2]
    per_row = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=2)[:, :, :S]
    return e4m3_decode(codes) * per_row[..., None]
