"""Rows that put the quantise-on-append codes at their rounding boundaries
(test input construction, shared by the GPU parity test and the CPU check of
the margin argument)."""

import numpy as np
import torch

import oracle


def boundary_rows(fmt, in_dtype, n_rows, seed):
    """Rows of 128 values whose first entry fixes the row's absmax (so the
    scale sc = fp16(absmax / QMAX) is known) and whose other 127 entries sit on
    or next to the code's rounding boundaries t * sc: int8 half-integers
    k + 1/2, fp8 midpoints between neighbouring E4M3 values, and QMAX itself;
    each rounded to the input type and moved by -2..2 of its units in the last
    place.  A third of the anchors make sc a power of two, so that many
    entries are exact ties."""
    rng = np.random.default_rng(seed)
    qmax = 127.0 if fmt == "int8" else 448.0
    if fmt == "int8":
        bnd = np.arange(127) + 0.5
    else:
        vals = np.unique(np.abs(oracle.dequant_fp8_fp64(np.arange(256, dtype=np.uint8)[None, :], np.ones(1))[0]))
        vals = vals[np.isfinite(vals) & (vals <= 448.0)]
        bnd = (vals[1:] + vals[:-1]) / 2
    bnd = np.concatenate([bnd, [qmax]])
    tdt = in_dtype
    e = rng.integers(-12, 8 if fmt == "int8" else 6, n_rows).astype(np.float64)  # anchors below fp16's max
    mant = np.where(rng.random(n_rows) < 1 / 3, 1.0, 1.0 + rng.integers(1, 128, n_rows) / 128.0)
    anchor = torch.from_numpy(qmax * mant * np.exp2(e)).to(tdt).double().numpy()
    sc = (anchor.astype(np.float32) / np.float32(qmax)).astype(np.float16).astype(np.float64)
    t = bnd[rng.integers(0, len(bnd), (n_rows, 127))]
    target = torch.from_numpy(t * sc[:, None]).to(tdt)
    bits = target.view(torch.int16).numpy().astype(np.int32)
    bits = bits + rng.integers(-2, 3, bits.shape)          # magnitudes are positive here
    mag = torch.from_numpy(bits.astype(np.int16)).view(tdt).double().numpy()
    mag = np.minimum(mag, anchor[:, None])                  # the anchor stays the absmax
    sign = np.where(rng.random(mag.shape) < 0.5, -1.0, 1.0)
    rows = np.concatenate([anchor[:, None], sign * mag], axis=1)
    return torch.from_numpy(rows).to(tdt)
