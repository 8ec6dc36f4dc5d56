"""Pins of the oracle's fp8 prefill-input quantiser (64-row power-of-two block scales) and
its random-sign Hadamard rotation: the rotation against scipy's Hadamard
matrix and its closed forms and invariances, the block quantiser against
torch's float8_e4m3fn cast and its error bound, and planted mistakes.  CPU only."""

from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle.quant import FP8_BLOCK_ROWS


def _signs(seed, d=128):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def test_rotation_matches_the_hadamard_matrix():
    x = np.random.default_rng(1).standard_normal((3, 5, 128)).astype(np.float32)
    s = _signs(2)
    y = oracle.hadamard_rotate_fp32(x, s)
    ref = (x.astype(np.float64) * s) @ scipy.linalg.hadamard(128) / math.sqrt(128)
    assert y.dtype == np.float32
    assert np.max(np.abs(y - ref)) < 1e-6 * np.max(np.abs(ref))


def test_rotation_closed_forms_and_invariances():
    s = _signs(3)
    # a unit vector e_i goes to row i of diag(s) H / sqrt(d), exactly
    e = np.zeros((128, 128), dtype=np.float32)
    np.fill_diagonal(e, 1.0)
    y = oracle.hadamard_rotate_fp32(e, s)
    want = (s[:, None] * scipy.linalg.hadamard(128)).astype(np.float32) * np.float32(1 / math.sqrt(128))
    assert np.array_equal(y, want)
    # orthogonal: norms kept, and Q K^T unchanged
    q = np.random.default_rng(4).standard_normal((7, 128)).astype(np.float32)
    k = np.random.default_rng(5).standard_normal((9, 128)).astype(np.float32)
    qr, kr = oracle.hadamard_rotate_fp32(q, s), oracle.hadamard_rotate_fp32(k, s)
    assert np.max(np.abs(np.linalg.norm(qr, axis=1) - np.linalg.norm(q, axis=1))) < 1e-5
    assert np.max(np.abs(qr.astype(np.float64) @ kr.T - q.astype(np.float64) @ k.T)) < 1e-4
    # an outlier channel is spread over all channels
    x = np.random.default_rng(6).standard_normal((1, 128)).astype(np.float32)
    x[0, 17] = 200.0
    assert np.max(np.abs(oracle.hadamard_rotate_fp32(x, s))) < 200.0 / math.sqrt(128) + 4.0


def test_block_quantiser_matches_torch_cast_and_bounds():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(2, 3, 150, 128, generator=g)
    x[0, 0, 70] *= 8.0  # an outlier row in the second block
    x[1, 2, 128:] = 0.0  # an all-zero (ragged) last block
    xb = x.to(torch.bfloat16)
    codes, scales = oracle.quantize_fp8_blocks(xb)
    assert codes.shape == (2, 3, 150, 128) and scales.shape == (2, 3, 3)
    xf = xb.float()
    for blk in range(3):
        r0, r1 = 64 * blk, min(150, 64 * blk + 64)
        part = xf[:, :, r0:r1]
        amax = part.abs().amax(dim=(2, 3))
        q = (amax / 448.0).numpy().astype(np.float32)
        s = scales[:, :, blk]
        # a power of two in [absmax/448, 2 absmax/448), or 0 for a zero block
        live = q > 0
        assert np.all(s[~live] == 0)
        mant, _ = np.frexp(s[live])
        assert np.all(mant == 0.5) and np.all(s[live] >= q[live]) and np.all(s[live] < 2 * q[live])
        safe = torch.from_numpy(np.where(s > 0, s, 1.0).astype(np.float32))
        ref = (part / safe[:, :, None, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ref = np.where((s > 0)[:, :, None, None], ref, 0)
        assert np.array_equal(codes[:, :, r0:r1], ref)
    assert np.all(codes[1, 2, 128:] == 0) and scales[1, 2, 2] == 0
    # the absmax element of each live block is +-448; the error within half a step
    deq = oracle.dequant_fp8_blocks_fp64(codes, scales)
    y = np.abs(xf.double().numpy()) / np.repeat(np.where(scales > 0, scales, 1), 64, axis=2)[:, :, :150, None]
    e = np.clip(np.floor(np.log2(np.where(y > 0, y, 1))), -6, 8)
    step = np.repeat(scales.astype(np.float64), 64, axis=2)[:, :, :150, None]
    assert np.all(np.abs(xf.double().numpy() - deq) <= (np.exp2(e - 4) + y * 2e-7) * step + 1e-30)
    # the absmax element of a live block lands in [224, 448]
    top = int(codes[0, 0, 64:128].reshape(-1)[np.argmax(np.abs(xf[0, 0, 64:128].numpy()).reshape(-1))])
    assert 224.0 <= abs(oracle.e4m3_decode(np.array([top], dtype=np.uint8))[0]) <= 448.0


def test_rotated_quantisation_reduces_channel_outlier_error():
    # with one outlier channel, per-block codes of rotated rows reproduce the
    # scores Q K^T better than codes of the rows themselves
    g = torch.Generator().manual_seed(8)
    q = torch.randn(1, 1, 64, 128, generator=g)
    k = torch.randn(1, 1, 64, 128, generator=g)
    k[..., 5] *= 60.0
    exact = q.double()[0, 0] @ k.double()[0, 0].T
    s = _signs(9)
    errs = []
    for signs in (None, s):
        qc, qs = oracle.quantize_fp8_blocks(q, signs)
        kc, ks = oracle.quantize_fp8_blocks(k, signs)
        approx = oracle.dequant_fp8_blocks_fp64(qc, qs)[0, 0] @ oracle.dequant_fp8_blocks_fp64(kc, ks)[0, 0].T
        errs.append(np.max(np.abs(approx - exact.numpy())))
    assert errs[1] < errs[0]


@pytest.mark.parametrize("kind", ["swapped_butterfly", "no_normalisation", "block_63", "per_tensor"])
def test_planted_fp8_quantiser_mistakes_are_caught(kind):
    g = torch.Generator().manual_seed(10)
    x = torch.randn(1, 2, 130, 128, generator=g)
    x[0, 0, 100] *= 6.0
    x[0, 1, 63] *= 5.0  # the last row of the first 64-row block
    s = _signs(11)
    caught = False
    # rotation mistakes: against the Hadamard matrix
    xf = x.numpy()[0, 0, :4]
    y = oracle.hadamard_rotate_fp32(xf, s)
    if kind == "swapped_butterfly":
        y = y.copy()
        y[:, [0, 1]] = y[:, [1, 0]]
    if kind == "no_normalisation":
        y = y * np.float32(math.sqrt(128))
    ref = (xf.astype(np.float64) * s) @ scipy.linalg.hadamard(128) / math.sqrt(128)
    caught |= bool(np.max(np.abs(y - ref)) > 1e-5)
    # block mistakes: the scale of each 64-row block is its absmax / 448
    codes, scales = oracle.quantize_fp8_blocks(x)
    if kind == "block_63":
        codes, scales = oracle.quantize_fp8_blocks(x, block_rows=63)
    if kind == "per_tensor":
        amax = float(x.abs().max())
        scales = np.full((1, 2, 3), oracle.quant.pow2_at_or_above(np.float32(amax / 448)), dtype=np.float32)
    q = np.stack([x[:, :, 64 * b:64 * b + 64].abs().amax(dim=(2, 3)).numpy() / 448 for b in range(3)], axis=-1)
    caught |= scales.shape != q.shape or bool(np.any(scales < q) or np.any(scales >= 2 * q))
    assert caught, kind


def test_pow2_at_or_above_closed_forms():
    f = oracle.quant.pow2_at_or_above
    v = np.array([1.0, 0.75, 0.5, 3.0, 2.0 ** -130, 1e-45, 0.0, 6.1e4], dtype=np.float32)
    want = np.array([1.0, 1.0, 0.5, 4.0, 2.0 ** -130, 2.0 ** -149, 0.0, 65536.0], dtype=np.float32)
    assert np.array_equal(f(v), want)
