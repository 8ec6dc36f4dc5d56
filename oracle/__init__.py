"""CPU oracle for exact tiled attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package. The GPU library never calls it, and it shares
no code with the GPU library: no kernels, headers, helpers or constants.

What it computes is the textbook definition that the FlashAttention pages say the
tiled method reproduces exactly (FlashAttention interview canvas, panel 1, the
"standard attention" and "one-sentence answer" boxes): S = Q K^T (scaled),
P = softmax(S) row by row, O = P V, plus the per-row log-sum-exp that the forward
keeps for recomputation (same page, panel 3, Q3). Everything is evaluated in
float64, two-pass (max first, then the normalised sum), with no tiling.

Modules
  attention  numpy float64 two-pass oracle (prefill, decode over a quantised
             cache), plus the pages' own online-softmax recurrence and a
             split-and-merge evaluation used only to pin invariants.
  backward   float64 gradients of attention (dQ, dK, dV given dO) from the
             softmax Jacobian, for the recomputing backward.
  brute      pure-Python scalar loops (math.exp / math.fsum) for tiny shapes.
  e4m3       OCP E4M3FN byte decoder written from the format's definition.
  quant      the KV-cache write side: per-token-per-head int8 and E4M3FN
             quantisers (and the E4M3FN encoder), and the append of quantised
             rows into a cache; the block-scaled fp8 quantiser of prefill
             inputs with optional random-sign Hadamard rotation.

Every function has a pin in tests/test_oracle.py, tests/test_oracle_kv.py or
tests/test_oracle_bwd.py
(brute force, closed forms, invariants, library special cases, a hand-derived
golden example); none of them is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_fp64,
    attention_probs_fp64,
    decode_fp64,
    dequant_fp8_fp64,
    dequant_int8_fp64,
    online_softmax_fp64,
    split_merge_fp64,
    visible_keys,
)
from .backward import attention_bwd_fp64  # noqa: F401
from .brute import attention_brute  # noqa: F401
from .e4m3 import e4m3_decode  # noqa: F401
from .quant import (  # noqa: F401
    dequant_fp8_blocks_fp64,
    e4m3_encode,
    hadamard_rotate_fp32,
    kv_append_ref,
    quantize_fp8_blocks,
    quantize_kv_tokhead,
)
