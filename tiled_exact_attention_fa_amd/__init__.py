"""Python binding of libfa, the MI355X exact tiled attention library.

Argument marshalling only: each function below has the name of the C entry
point it calls (declared in include/fa.h), turns torch tensors into device
pointers and element strides, passes torch's current HIP stream, and raises
FaError on a negative status.  Every step of the computation runs in the HIP
kernels of libfa.so; there is no fallback of any kind — if the library has not
been built, load() raises.

    fa_fwd(q, k, v, o, lse=None, causal=False, softmax_scale=None, ...)
    fa_decode_kvq(q, k_cache, v_cache, k_scale, v_scale, o, lse=None, ...)
    fa_decode_kvq_noalloc(...)  (no workspace: the library's fixed per-GPU scratch)
    fa_decode_workspace_size(B, Hq, d, num_splits)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=False, ...)
    fa_bwd_workspace_size(B, Hq, Sq)
    fa_fp8_quantize(x, codes, scales, signs=None)
    fa_kv_append(k_new, v_new, k_cache, v_cache, k_scale, v_scale, positions=None, ...)
    fa_check_fwd_params(params) / fa_check_bwd_params(params) /
    fa_check_decode_params(params) / fa_check_kv_append_params(params) /
    fa_check_fp8_quant_params(params)
    fa_status_string(status) / fa_last_error()

Build with ``python -m tiled_exact_attention_fa_amd.build``.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3, FA_INT8 = 0, 1, 2, 3, 4
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGNMENT, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, -1, -2, -3, -4, -5
FA_KV_INT8_TOKHEAD_F16SCALE, FA_KV_FP8_E4M3_TOKHEAD_F16SCALE = 0, 1

I64x3 = ctypes.c_int64 * 3
I64x2 = ctypes.c_int64 * 2


class FaFwdParams(ctypes.Structure):
    """Mirror of fa_fwd_params."""

    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_strides", I64x3), ("k_strides", I64x3), ("v_strides", I64x3), ("o_strides", I64x3),
        ("lse_strides", I64x2),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
        ("q_block_descale", ctypes.c_void_p), ("k_block_descale", ctypes.c_void_p),
        ("v_block_descale", ctypes.c_void_p),
        ("fp8_p_bf16", ctypes.c_int32), ("soft_exp2", ctypes.c_int32),
    ]


class FaFp8QuantParams(ctypes.Structure):
    """Mirror of fa_fp8_quant_params."""

    _fields_ = [
        ("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("signs", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("x_strides", I64x3), ("codes_strides", I64x3),
    ]


class FaDecodeParams(ctypes.Structure):
    """Mirror of fa_decode_params."""

    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("L", ctypes.c_int32),
        ("d", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("q_strides", I64x2), ("kv_strides", I64x3), ("scale_strides", I64x2),
        ("o_strides", I64x2), ("lse_strides", I64x2),
        ("kv_format", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("k_recent", ctypes.c_void_p), ("v_recent", ctypes.c_void_p), ("recent_lens", ctypes.c_void_p),
        ("W", ctypes.c_int32), ("recent_strides", I64x3),
    ]


class FaBwdParams(ctypes.Structure):
    """Mirror of fa_bwd_params."""

    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_strides", I64x3), ("k_strides", I64x3), ("v_strides", I64x3), ("o_strides", I64x3),
        ("do_strides", I64x3), ("dq_strides", I64x3), ("dk_strides", I64x3), ("dv_strides", I64x3),
        ("lse_strides", I64x2),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("wave_pingpong", ctypes.c_int32),
    ]


class FaKvAppendParams(ctypes.Structure):
    """Mirror of fa_kv_append_params."""

    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("positions", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int32), ("kv_format", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("L", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("new_strides", I64x3), ("kv_strides", I64x3), ("scale_strides", I64x2),
    ]


FA_DECODE_NOALLOC_MAX_BYTES = 32 * 1024 * 1024

EXPORTS = ["fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_decode_kvq", "fa_decode_kvq_noalloc",
           "fa_decode_workspace_size",
           "fa_kv_append", "fa_fp8_quantize", "fa_check_fwd_params", "fa_check_bwd_params",
           "fa_check_decode_params", "fa_check_kv_append_params", "fa_check_fp8_quant_params",
           "fa_status_string", "fa_last_error"]


class FaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {fa_status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None


def load(path: str | None = None):
    """Loads libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m tiled_exact_attention_fa_amd.build`")
    lib = ctypes.CDLL(p)
    lib.fa_fwd.argtypes = [ctypes.POINTER(FaFwdParams), ctypes.c_void_p]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_decode_kvq.argtypes = [ctypes.POINTER(FaDecodeParams), ctypes.c_void_p]
    lib.fa_decode_kvq.restype = ctypes.c_int
    lib.fa_decode_kvq_noalloc.argtypes = [ctypes.POINTER(FaDecodeParams), ctypes.c_void_p]
    lib.fa_decode_kvq_noalloc.restype = ctypes.c_int
    lib.fa_decode_workspace_size.argtypes = [ctypes.c_int32] * 4
    lib.fa_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_check_fwd_params.argtypes = [ctypes.POINTER(FaFwdParams)]
    lib.fa_check_fwd_params.restype = ctypes.c_int
    lib.fa_check_decode_params.argtypes = [ctypes.POINTER(FaDecodeParams)]
    lib.fa_check_decode_params.restype = ctypes.c_int
    lib.fa_fp8_quantize.argtypes = [ctypes.POINTER(FaFp8QuantParams), ctypes.c_void_p]
    lib.fa_fp8_quantize.restype = ctypes.c_int
    lib.fa_check_fp8_quant_params.argtypes = [ctypes.POINTER(FaFp8QuantParams)]
    lib.fa_check_fp8_quant_params.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [ctypes.POINTER(FaBwdParams), ctypes.c_void_p]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_check_bwd_params.argtypes = [ctypes.POINTER(FaBwdParams)]
    lib.fa_check_bwd_params.restype = ctypes.c_int
    lib.fa_bwd_workspace_size.argtypes = [ctypes.c_int32] * 3
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_kv_append.argtypes = [ctypes.POINTER(FaKvAppendParams), ctypes.c_void_p]
    lib.fa_kv_append.restype = ctypes.c_int
    lib.fa_check_kv_append_params.argtypes = [ctypes.POINTER(FaKvAppendParams)]
    lib.fa_check_kv_append_params.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def fa_check_fwd_params(params: FaFwdParams) -> int:
    return load().fa_check_fwd_params(ctypes.byref(params))


def fa_check_decode_params(params: FaDecodeParams) -> int:
    return load().fa_check_decode_params(ctypes.byref(params))


def fa_check_fp8_quant_params(params: FaFp8QuantParams) -> int:
    return load().fa_check_fp8_quant_params(ctypes.byref(params))


def fa_check_bwd_params(params: FaBwdParams) -> int:
    return load().fa_check_bwd_params(ctypes.byref(params))


def fa_bwd_workspace_size(B: int, Hq: int, Sq: int) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, Sq))


def fa_check_kv_append_params(params: FaKvAppendParams) -> int:
    return load().fa_check_kv_append_params(ctypes.byref(params))


def fa_decode_workspace_size(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(load().fa_decode_workspace_size(B, Hq, d, num_splits))


# ---- torch marshalling -------------------------------------------------------

def _dtype_code(t) -> int:
    import torch

    table = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16,
             torch.float8_e4m3fn: FA_FP8_E4M3, torch.int8: FA_INT8}
    if t.dtype not in table:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return table[t.dtype]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require_dense_d(name, t):
    if t is not None and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last (head) dimension must have stride 1")


# The C ABI sees pointers and the sizes taken from q and k only, so every other
# tensor is checked here against them: a shorter o or v, a bf16 lse or an int64
# seq_lens would otherwise be read or written past its end by the kernels.

def _dims(name, t, n):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != n:
        raise ValueError(f"{name}: expected {n} dimensions, got shape {tuple(t.shape)}")


def _expect(name, t, shape, dtypes):
    """t has exactly `shape` and one of `dtypes` (a torch dtype or a tuple)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")


def _expect_vector(name, t, n, dtype):
    """A contiguous 1-D tensor of n elements of `dtype` (per-sequence lengths,
    positions, rotation signs)."""
    _expect(name, t, (n,), dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _unit_last_stride(name, t):
    if t is not None and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must have stride 1")


def _same_gpu(**tensors):
    """Every given tensor lives on one GPU: a host pointer handed to a kernel
    would fault the device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} is not on a GPU (device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def fwd_params(q, k, v, o, lse=None, causal=False, softmax_scale=None,
               q_descale=1.0, k_descale=1.0, v_descale=1.0, block_descales=None,
               p_bf16=False, soft_exp2=False) -> FaFwdParams:
    """fa_fwd_params for BHSD-indexed tensors q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d]
    (q's dtype), o [B,Hq,Sq,d] (q's dtype, bf16 for fp8 inputs), lse [B,Hq,Sq]
    float32 (any strides with a unit last stride), all on one GPU.  p_bf16
    sets fp8_p_bf16 (fp8 inputs only), soft_exp2 the software-exponential
    split (bf16/fp16, d = 128)."""
    import torch

    _dims("q", q, 4)
    _dims("k", k, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    out_dt = {torch.float32: torch.float32, torch.float16: torch.float16, torch.bfloat16: torch.bfloat16,
              torch.float8_e4m3fn: torch.bfloat16}.get(q.dtype)
    if out_dt is None:
        raise TypeError(f"q: dtype {q.dtype} is not an fa_fwd input type")
    _expect("k", k, (B, Hkv, Sk, d), q.dtype)
    _expect("v", v, (B, Hkv, Sk, d), q.dtype)
    _expect("o", o, (B, Hq, Sq, d), out_dt)
    if lse is not None:
        _expect("lse", lse, (B, Hq, Sq), torch.float32)
        _unit_last_stride("lse", lse)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _require_dense_d(n, t)
    if block_descales is not None:
        if len(block_descales) != 3:
            raise ValueError("block_descales is a (q, k, v) triple")
        for n, t, rows in zip(("q", "k", "v"), block_descales, (Sq, Sk, Sk)):
            _expect(f"{n} block descales", t, (B, Hq if n == "q" else Hkv, (rows + 63) // 64), torch.float32)
            if not t.is_contiguous():
                raise ValueError("block descales must be contiguous")
    bd = block_descales or (None, None, None)
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse, q_block_descale=bd[0], k_block_descale=bd[1], v_block_descale=bd[2])
    p = FaFwdParams()
    p.q, p.k, p.v, p.o, p.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    p.in_dtype, p.out_dtype = _dtype_code(q), _dtype_code(o)
    p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.d = B, Hq, Hkv, Sq, Sk, d
    p.q_strides = I64x3(*q.stride()[:3])
    p.k_strides = I64x3(*k.stride()[:3])
    p.v_strides = I64x3(*v.stride()[:3])
    p.o_strides = I64x3(*o.stride()[:3])
    p.lse_strides = I64x2(*(lse.stride()[:2] if lse is not None else (0, 0)))
    p.softmax_scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    p.causal = 1 if causal else 0
    p.q_descale, p.k_descale, p.v_descale = float(q_descale), float(k_descale), float(v_descale)
    if block_descales is not None:  # (q, k, v) float32 tensors [B, H, ceil(S / 64)], contiguous
        p.q_block_descale, p.k_block_descale, p.v_block_descale = (_ptr(t) for t in block_descales)
    p.fp8_p_bf16 = 1 if p_bf16 else 0
    p.soft_exp2 = 1 if soft_exp2 else 0
    return p


def fa_fwd(q, k, v, o, lse=None, causal=False, softmax_scale=None,
           q_descale=1.0, k_descale=1.0, v_descale=1.0, stream=None, block_descales=None,
           p_bf16=False, soft_exp2=False) -> None:
    """Enqueue the prefill forward on torch's current stream (or ``stream``).
    ``block_descales``: optional (q, k, v) per-64-row descales for fp8 inputs;
    ``p_bf16``: fp8 inputs only, probabilities rounded to bf16 for P V instead
    of e4m3."""
    p = fwd_params(q, k, v, o, lse, causal, softmax_scale, q_descale, k_descale, v_descale, block_descales,
                   p_bf16, soft_exp2)
    st = load().fa_fwd(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd", fa_last_error())


def _kv_format(cache, kv_format):
    """fa_kv_format from an explicit name/code, else from the cache dtype:
    int8 -> int8 codes; float8_e4m3fn or uint8 -> E4M3FN bytes."""
    import torch

    if kv_format is not None:
        return {"int8": FA_KV_INT8_TOKHEAD_F16SCALE, "fp8": FA_KV_FP8_E4M3_TOKHEAD_F16SCALE}.get(kv_format, kv_format)
    if cache.dtype == torch.int8:
        return FA_KV_INT8_TOKHEAD_F16SCALE
    if cache.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FA_KV_FP8_E4M3_TOKHEAD_F16SCALE
    raise TypeError(f"cannot infer the cache format from dtype {cache.dtype}")


def fp8_quant_params(x, codes, scales, signs=None) -> FaFp8QuantParams:
    """fa_fp8_quant_params for x [B,H,S,d] bf16/fp16, codes [B,H,S,d] uint8 or
    float8_e4m3fn, scales [B,H,ceil(S/64)] float32 contiguous, signs [d] float32."""
    import torch

    _dims("x", x, 4)
    B, H, S, d = x.shape
    _expect("x", x, (B, H, S, d), (torch.bfloat16, torch.float16))
    _expect("codes", codes, (B, H, S, d), (torch.uint8, torch.float8_e4m3fn))
    _expect("scales", scales, (B, H, (S + 63) // 64), torch.float32)
    if not scales.is_contiguous():
        raise ValueError("scales must be contiguous")
    if signs is not None:
        _expect_vector("signs", signs, d, torch.float32)
    _require_dense_d("x", x)
    _require_dense_d("codes", codes)
    _same_gpu(x=x, codes=codes, scales=scales, signs=signs)
    p = FaFp8QuantParams()
    p.x, p.codes, p.scales, p.signs = _ptr(x), _ptr(codes), _ptr(scales), _ptr(signs)
    p.in_dtype = _dtype_code(x)
    p.B, p.H, p.S, p.d = B, H, S, d
    p.x_strides = I64x3(*x.stride()[:3])
    p.codes_strides = I64x3(*codes.stride()[:3])
    return p


def fa_fp8_quantize(x, codes, scales, signs=None, stream=None) -> None:
    """Enqueue the block-scaled fp8 quantisation (optionally rotated) of x."""
    p = fp8_quant_params(x, codes, scales, signs)
    st = load().fa_fp8_quantize(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fp8_quantize", fa_last_error())


def bwd_params(q, k, v, o, dout, lse, dq, dk, dv, causal=False, softmax_scale=None,
               workspace=None, wave_pingpong=False) -> FaBwdParams:
    """fa_bwd_params for q/o/dout/dq [B,Hq,Sq,d], k/v/dk/dv [B,Hkv,Sk,d] and
    lse [B,Hq,Sq] float32 (any strides with a unit head-dim stride);
    wave_pingpong selects the dK/dV kernel's wave-specialised schedule."""
    import torch

    _dims("q", q, 4)
    _dims("k", k, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"q: dtype {q.dtype}, expected torch.bfloat16 or torch.float16")
    for n, t in (("o", o), ("dout", dout), ("dq", dq)):
        _expect(n, t, (B, Hq, Sq, d), q.dtype)
    for n, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _expect(n, t, (B, Hkv, Sk, d), q.dtype)
    _expect("lse", lse, (B, Hq, Sq), torch.float32)
    _unit_last_stride("lse", lse)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _require_dense_d(n, t)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    p = FaBwdParams()
    p.q, p.k, p.v, p.o, p.dout, p.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse)
    p.dq, p.dk, p.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    p.dtype = _dtype_code(q)
    p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.d = B, Hq, Hkv, Sq, Sk, d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(p, f"{name}_strides", I64x3(*t.stride()[:3]))
    p.lse_strides = I64x2(*lse.stride()[:2])
    p.softmax_scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    p.causal = 1 if causal else 0
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.wave_pingpong = 1 if wave_pingpong else 0
    return p


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, causal=False, softmax_scale=None, workspace=None,
           stream=None, wave_pingpong=False) -> None:
    """Enqueue the backward (dq, dk, dv from dout, o and the forward's lse)."""
    import torch

    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_size(q.shape[0], q.shape[1], q.shape[2]),
                                dtype=torch.uint8, device=q.device)
    p = bwd_params(q, k, v, o, dout, lse, dq, dk, dv, causal, softmax_scale, workspace, wave_pingpong)
    st = load().fa_bwd(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd", fa_last_error())


def decode_params(q, k_cache, v_cache, k_scale, v_scale, o, lse=None, seq_lens=None,
                  num_splits=16, softmax_scale=None, workspace=None, kv_format=None,
                  k_recent=None, v_recent=None, recent_lens=None) -> FaDecodeParams:
    """fa_decode_params for q [B,Hq,d], caches [B,Hkv,L,d], scales [B,Hkv,L],
    o [B,Hq,d], lse [B,Hq], and an optional bf16 window k_recent/v_recent
    [B,Hkv,W,d]; k and v caches (and their scales, and the two window tensors)
    must share strides."""
    import torch

    _dims("q", q, 3)
    _dims("k_cache", k_cache, 4)
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    codes = (torch.int8, torch.uint8, torch.float8_e4m3fn)
    _expect("q", q, (B, Hq, d), torch.bfloat16)
    _expect("k_cache", k_cache, (B, Hkv, L, d), codes)
    _expect("v_cache", v_cache, (B, Hkv, L, d), k_cache.dtype)
    _expect("k_scale", k_scale, (B, Hkv, L), torch.float16)
    _expect("v_scale", v_scale, (B, Hkv, L), torch.float16)
    _expect("o", o, (B, Hq, d), torch.bfloat16)
    if lse is not None:
        _expect("lse", lse, (B, Hq), torch.float32)
    if seq_lens is not None:
        _expect_vector("seq_lens", seq_lens, B, torch.int32)
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("o", o),
                 ("k_scale", k_scale), ("v_scale", v_scale), ("k_recent", k_recent), ("v_recent", v_recent)):
        _require_dense_d(n, t)
    if k_cache.stride() != v_cache.stride() or k_scale.stride() != v_scale.stride():
        raise ValueError("k and v caches (and their scales) must have identical strides")
    if (k_recent is None) != (v_recent is None):
        raise ValueError("k_recent and v_recent go together")
    if k_recent is not None:
        _dims("k_recent", k_recent, 4)
        W = k_recent.shape[2]
        _expect("k_recent", k_recent, (B, Hkv, W, d), torch.bfloat16)
        _expect("v_recent", v_recent, (B, Hkv, W, d), torch.bfloat16)
        if k_recent.stride() != v_recent.stride():
            raise ValueError("k_recent and v_recent must have identical strides")
        if recent_lens is not None:
            _expect_vector("recent_lens", recent_lens, B, torch.int32)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_gpu(q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, o=o, lse=lse,
              seq_lens=seq_lens, workspace=workspace, k_recent=k_recent, v_recent=v_recent,
              recent_lens=recent_lens if k_recent is not None else None)
    p = FaDecodeParams()
    p.q, p.k_cache, p.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    p.k_scale, p.v_scale, p.seq_lens = _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens)
    p.o, p.lse = _ptr(o), _ptr(lse)
    p.B, p.Hq, p.Hkv, p.L, p.d, p.num_splits = B, Hq, Hkv, L, d, int(num_splits)
    p.q_strides = I64x2(*q.stride()[:2])
    p.kv_strides = I64x3(*k_cache.stride()[:3])
    p.scale_strides = I64x2(*k_scale.stride()[:2])
    p.o_strides = I64x2(*o.stride()[:2])
    p.lse_strides = I64x2(*(lse.stride()[:2] if lse is not None else (0, 0)))
    p.kv_format = _kv_format(k_cache, kv_format)
    p.softmax_scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if k_recent is not None:
        p.k_recent, p.v_recent, p.recent_lens = _ptr(k_recent), _ptr(v_recent), _ptr(recent_lens)
        p.W = k_recent.shape[2]
        p.recent_strides = I64x3(*k_recent.stride()[:3])
    return p


def decode_workspace(B, Hq, d, num_splits, device="cuda", window=False):
    """A torch byte tensor big enough for fa_decode_kvq's partial results
    (one more partial slot when a residual window is used)."""
    import torch

    n = fa_decode_workspace_size(B, Hq, d, num_splits + (1 if window else 0))
    return torch.empty(n, dtype=torch.uint8, device=device)


def fa_decode_kvq(q, k_cache, v_cache, k_scale, v_scale, o, lse=None, seq_lens=None,
                  num_splits=16, softmax_scale=None, workspace=None, stream=None, kv_format=None,
                  k_recent=None, v_recent=None, recent_lens=None) -> None:
    """Enqueue one decode step over the quantised cache (and the optional bf16
    residual window) on torch's current stream."""
    if workspace is None:
        workspace = decode_workspace(q.shape[0], q.shape[1], q.shape[2], num_splits, q.device,
                                     window=k_recent is not None and k_recent.shape[2] > 0)
    p = decode_params(q, k_cache, v_cache, k_scale, v_scale, o, lse, seq_lens, num_splits,
                      softmax_scale, workspace, kv_format, k_recent, v_recent, recent_lens)
    st = load().fa_decode_kvq(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_decode_kvq", fa_last_error())


def kv_append_params(k_new, v_new, k_cache, v_cache, k_scale, v_scale, positions=None,
                     kv_format=None) -> FaKvAppendParams:
    """fa_kv_append_params for new rows k_new/v_new [B,H,T,d] (bf16 or fp16),
    caches [B,H,L,d] and scales [B,H,L]; positions [B] int32 or None."""
    import torch

    _dims("k_new", k_new, 4)
    _dims("k_cache", k_cache, 4)
    B, H, T, d = k_new.shape
    L = k_cache.shape[2]
    _expect("k_new", k_new, (B, H, T, d), (torch.bfloat16, torch.float16))
    _expect("v_new", v_new, (B, H, T, d), k_new.dtype)
    _expect("k_cache", k_cache, (B, H, L, d), (torch.int8, torch.uint8, torch.float8_e4m3fn))
    _expect("v_cache", v_cache, (B, H, L, d), k_cache.dtype)
    _expect("k_scale", k_scale, (B, H, L), torch.float16)
    _expect("v_scale", v_scale, (B, H, L), torch.float16)
    if positions is not None:
        _expect_vector("positions", positions, B, torch.int32)
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("k_scale", k_scale), ("v_scale", v_scale)):
        _require_dense_d(n, t)
    if k_new.stride() != v_new.stride() or k_cache.stride() != v_cache.stride() \
            or k_scale.stride() != v_scale.stride():
        raise ValueError("k and v tensors of each kind must have identical strides")
    _same_gpu(k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
              positions=positions)
    p = FaKvAppendParams()
    p.k_new, p.v_new = _ptr(k_new), _ptr(v_new)
    p.k_cache, p.v_cache = _ptr(k_cache), _ptr(v_cache)
    p.k_scale, p.v_scale = _ptr(k_scale), _ptr(v_scale)
    p.positions = _ptr(positions)
    p.in_dtype = _dtype_code(k_new)
    p.kv_format = _kv_format(k_cache, kv_format)
    p.B, p.H, p.T, p.L, p.d = B, H, T, k_cache.shape[2], d
    p.new_strides = I64x3(*k_new.stride()[:3])
    p.kv_strides = I64x3(*k_cache.stride()[:3])
    p.scale_strides = I64x2(*k_scale.stride()[:2])
    return p


def fa_kv_append(k_new, v_new, k_cache, v_cache, k_scale, v_scale, positions=None,
                 kv_format=None, stream=None) -> None:
    """Enqueue the quantise-on-append of new key/value rows into the cache."""
    p = kv_append_params(k_new, v_new, k_cache, v_cache, k_scale, v_scale, positions, kv_format)
    st = load().fa_kv_append(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_kv_append", fa_last_error())


def fa_decode_kvq_noalloc(q, k_cache, v_cache, k_scale, v_scale, o, lse=None, seq_lens=None,
                          num_splits=16, softmax_scale=None, stream=None, kv_format=None,
                          k_recent=None, v_recent=None, recent_lens=None) -> None:
    """fa_decode_kvq without a workspace: the split partials go to the
    library's fixed per-GPU scratch (FA_DECODE_NOALLOC_MAX_BYTES), so nothing
    is allocated; concurrent calls on one GPU race on it."""
    p = decode_params(q, k_cache, v_cache, k_scale, v_scale, o, lse, seq_lens, num_splits,
                      softmax_scale, None, kv_format, k_recent, v_recent, recent_lens)
    st = load().fa_decode_kvq_noalloc(ctypes.byref(p), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_decode_kvq_noalloc", fa_last_error())
