"""OCP FP8 E4M3FN decoder — TEST INFRASTRUCTURE ONLY.

The FlashAttention-3 page (Hopper asynchrony, "new bottleneck on Hopper" box)
names FP8 as a throughput lever whose error must be controlled; the format used
here is OCP E4M3FN, the FP8 format that gfx950 matrix cores read: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, and the two codes
with every exponent and mantissa bit set (0x7F, 0xFF) are NaN.  Largest finite
magnitude 1.75 * 2^8 = 448; exponent field 0 encodes subnormals m/8 * 2^-6.

Written from that definition; it shares nothing with the GPU path.
"""

from __future__ import annotations

import math

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN byte."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Decode an array of E4M3FN bytes (uint8/int8 numpy, or a torch tensor of
    dtype uint8/int8/float8_e4m3fn) into float64."""
    if not isinstance(codes, np.ndarray):
        import torch

        t = codes.detach().to("cpu")
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8) if t.element_size() == 1 else t.to(torch.uint8)
        codes = t.numpy()
    return _TABLE[codes.astype(np.uint8)]
