"""Float64 two-pass attention oracle — TEST INFRASTRUCTURE ONLY (see package doc).

Definitions follow the pages:

* Standard attention (FlashAttention interview canvas, panel 1, "standard
  attention" box): scores S = Q K^T, probabilities P = softmax(S) per row,
  output O = P V.  The tiled method is stated to be exact, with no approximation
  (same panel, "one-sentence answer" box), so this plain definition is the oracle.
* Per-row statistic kept by the forward pass (same page, panel 3, Q3): the
  log-sum-exp LSE_i = m_i + ln l_i, natural log.
* Online-softmax state m / l / O and the exp(old_m - new_m) rescale (same page,
  panel 1 "online softmax key state" box and panel 3, Q2) — used only by
  ``online_softmax_fp64``, the pages' recurrence, to pin the exactness claim.
* Decode over a quantised cache (KV-cache quantisation overview, section 1 "decode
  step" and section 3 "read path"): one new query attends to every cached key;
  the cache is dequantised into the compute domain (int8 or E4M3FN code x
  per-token scale).  The optional residual window (same section, "residual
  window" box: the most recent tokens stay in high precision) adds bf16 keys and
  values that are attended next to the dequantised ones.

Readings where the pages are silent (each is listed in the design notes):
  scale tau = 1/sqrt(d) unless given; causal mask is bottom-right aligned (key j
  visible from query i iff j <= i + Sk - Sq); a row with no visible key has
  O = 0 and LSE = -inf; GQA maps query head h to kv head h // (Hq/Hkv).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep BLAS single-threaded inside the per-head worker pool
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover
    threadpool_limits = None


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 of a numpy array or a CPU torch tensor (bf16 too)."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    import torch  # only for the dtype conversion of bf16/fp16/fp8 tensors

    return x.detach().to("cpu").to(torch.float64).numpy()


def visible_keys(i: int, Sq: int, Sk: int, causal: bool) -> int:
    """Number of leading keys visible from query row i (keys 0..n-1).

    Causal reading: bottom-right aligned, key j visible iff j <= i + Sk - Sq.
    """
    if not causal:
        return Sk
    return int(min(Sk, max(0, i + Sk - Sq + 1)))


def _default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _two_pass_rows(qh, kh, vh, scale, n_vis, row_block):
    """Two-pass softmax attention for one (batch, head).

    qh [Sq,d], kh [Sk,d], vh [Sk,dv] float64; n_vis[i] = visible key count of row i.
    Pass 1: m_i = max_j s_ij and l_i = sum_j exp(s_ij - m_i) over visible j.
    Pass 2: O_i = sum_j exp(s_ij - m_i) / l_i * V_j ;  LSE_i = m_i + ln l_i.
    """
    Sq = qh.shape[0]
    o = np.zeros((Sq, vh.shape[1]), dtype=np.float64)
    lse = np.full((Sq,), -np.inf, dtype=np.float64)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        # keys past the block's last visible one are never evaluated: under the
        # mask they would enter only as exact zeros
        nk = int(n_vis[r0:r1].max(initial=0))
        s = (qh[r0:r1] @ kh[:nk].T) * scale  # [R, nk]
        vis = np.arange(nk)[None, :] < n_vis[r0:r1, None]
        s = np.where(vis, s, -np.inf)
        has = n_vis[r0:r1] > 0
        # pass 1: row max and normaliser
        m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(s - m[:, None]), 0.0)
        l = e.sum(axis=1)
        # pass 2: normalised probabilities times V
        p = e / np.where(has, l, 1.0)[:, None]
        o[r0:r1] = p @ vh[:nk]
        lse[r0:r1] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse


def attention_fp64(q, k, v, causal: bool = False, scale: float | None = None,
                   heads=None, row_block: int = 512, threads: int | None = None, rows=None):
    """Exact attention in float64.

    q [B,Hq,Sq,d]; k [B,Hkv,Sk,d]; v [B,Hkv,Sk,dv]; Hq % Hkv == 0.
    Returns (O [B,Hq,R,dv] float64, LSE [B,Hq,R] float64) with R = Sq, or
    R = len(rows) when ``rows`` lists the query rows to evaluate (absolute
    positions, so the causal rule is unchanged) — for sampled checks.
    ``heads``: optional iterable of (b, h) pairs; only those are computed (the
    other entries stay O = 0, LSE = -inf) — for sampled checks at full size.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    assert Bk == B and dk == d and v.shape[:3] == (B, Hkv, Sk)
    assert Hq % Hkv == 0
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    sel = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    n_vis = np.array([visible_keys(int(i), Sq, Sk, causal) for i in sel], dtype=np.int64)
    o = np.zeros((B, Hq, len(sel), v.shape[3]), dtype=np.float64)
    lse = np.full((B, Hq, len(sel)), -np.inf, dtype=np.float64)
    work = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        b, h = bh
        kvh = h // G
        o[b, h], lse[b, h] = _two_pass_rows(q[b, h][sel], k[b, kvh], v[b, kvh], tau, n_vis, row_block)

    nthreads = threads or _default_threads()
    if nthreads <= 1 or len(work) <= 1:
        for bh in work:
            one(bh)
    else:
        ctx = threadpool_limits(1) if threadpool_limits is not None else _Null()
        with ctx, ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one, work))
    return o, lse


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def attention_probs_fp64(q, k, causal: bool = False, scale: float | None = None):
    """The full probability matrix P [B,Hq,Sq,Sk] (tiny shapes only, for invariants)."""
    q = _f64(q)
    k = _f64(k)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    p = np.zeros((B, Hq, Sq, Sk), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s = (q[b, h] @ k[b, h // G].T) * tau
            for i in range(Sq):
                n = visible_keys(i, Sq, Sk, causal)
                if n == 0:
                    continue
                row = s[i, :n]
                e = np.exp(row - row.max())
                p[b, h, i, :n] = e / e.sum()
    return p


def online_softmax_fp64(q, k, v, causal: bool = False, scale: float | None = None,
                        block_q: int = 64, block_k: int = 64, trace: list | None = None):
    """The pages' tiled recurrence in float64, used to pin the exactness claim.

    Query rows are taken block_q at a time and keys block_k at a time.  For each
    key block the running state (m = running row max, l = rescaled sum of exps,
    O = un-normalised accumulator) is updated: the old O and l are multiplied by
    exp(old_m - new_m) and the new block's exp(s - new_m) terms are added
    (FlashAttention interview canvas, panel 1 "online softmax key state" box and
    panel 3, Q2).  The final O is divided by l (softmax definition) and
    LSE = m + ln l.  If ``trace`` is a list, the state (m, l, O) after every key
    block is appended to it as copies, for checking a hand-derived example.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    o = np.zeros((B, Hq, Sq, v.shape[3]))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, h // G], v[b, h // G]
            for r0 in range(0, Sq, block_q):
                r1 = min(Sq, r0 + block_q)
                nq = r1 - r0
                m = np.full(nq, -np.inf)
                l = np.zeros(nq)
                acc = np.zeros((nq, vv.shape[1]))
                n_vis = np.array([visible_keys(i, Sq, Sk, causal) for i in range(r0, r1)])
                for c0 in range(0, Sk, block_k):
                    c1 = min(Sk, c0 + block_k)
                    s = (q[b, h, r0:r1] @ kk[c0:c1].T) * tau
                    vis = np.arange(c0, c1)[None, :] < n_vis[:, None]
                    s = np.where(vis, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)
                    m_safe = np.where(live, m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - m_safe), 0.0)
                    p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ vv[c0:c1]
                    m = m_new
                    if trace is not None:
                        trace.append((m.copy(), l.copy(), acc.copy()))
                has = l > 0
                o[b, h, r0:r1] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse


def split_merge_fp64(q, k, v, num_splits: int, scale: float | None = None):
    """Non-causal attention evaluated as key chunks merged by their log-sum-exps.

    Keys are cut into num_splits equal chunks of ceil(Sk/num_splits) (the last may
    be short or empty).  Each chunk gives a normalised partial O_s and lse_s; they
    merge as LSE = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
    O = sum_s exp(lse_s - LSE) O_s — the same m/l algebra as the online-softmax
    rescale (FlashAttention interview canvas, panel 3, Q2), applied to whole
    chunks.  An empty chunk has lse_s = -inf and contributes nothing.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    Sk = k.shape[2]
    chunk = -(-Sk // num_splits)
    parts = []
    for s in range(num_splits):
        c0, c1 = s * chunk, min(Sk, (s + 1) * chunk)
        if c1 <= c0:
            shape = q.shape[:3]
            parts.append((np.zeros(shape + (v.shape[3],)), np.full(shape, -np.inf)))
            continue
        parts.append(attention_fp64(q, k[:, :, c0:c1], v[:, :, c0:c1], False, scale, threads=1))
    lses = np.stack([p[1] for p in parts])  # [S, B, H, Sq]
    M = lses.max(axis=0)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    w = np.exp(lses - Ms[None])
    tot = w.sum(axis=0)
    lse = np.where(live, Ms + np.log(np.where(live, tot, 1.0)), -np.inf)
    o = np.zeros(parts[0][0].shape)
    for s, (os_, ls) in enumerate(parts):
        coef = np.where(live, np.exp(ls - np.where(live, lse, 0.0)), 0.0)
        o += coef[..., None] * os_
    return o, lse


def dequant_int8_fp64(codes, scales) -> np.ndarray:
    """int8 code times its per-token fp16 scale, in float64 (exact).

    KV-cache quantisation overview, section 3 "read path": the stored low-bit
    value is mapped back into the compute domain with its scale.  Symmetric
    codes, so there is no zero point.  codes [..., T, d], scales [..., T].
    """
    return _f64(codes) * _f64(scales)[..., None]


def dequant_fp8_fp64(codes, scales) -> np.ndarray:
    """E4M3FN code (decoded by the oracle's own decoder) times its per-token
    fp16 scale, in float64 (exact: a 4-bit by 11-bit significand product).
    codes [..., T, d] as bytes, scales [..., T]."""
    from .e4m3 import e4m3_decode

    return e4m3_decode(codes) * _f64(scales)[..., None]


def _as_list(lens, B, default):
    if lens is None:
        return [default] * B
    return [int(x) for x in (lens.tolist() if hasattr(lens, "tolist") else lens)]


def decode_fp64(q, k_codes, k_scales, v_codes, v_scales, seq_lens=None,
                scale: float | None = None, heads=None, threads: int | None = None,
                kv_format: str = "int8", k_recent=None, v_recent=None, recent_lens=None):
    """One-token decode over a quantised cache with per-token-per-head fp16 scales.

    q [B,Hq,d]; k_codes/v_codes [B,Hkv,L,d] (int8 codes, or E4M3FN bytes when
    kv_format is "fp8"); k_scales/v_scales [B,Hkv,L].  seq_lens [B] or None
    (all L): each query row sees cache tokens 0..seq_len-1 (KV-cache
    quantisation overview, section 1: the decode step's new token queries every
    cached key).  With a residual window, k_recent/v_recent [B,Hkv,W,d] hold the
    most recent tokens unquantised and recent_lens [B] (None = all W) of them are
    attended as well; the window's keys join the same softmax.  Returns
    (O [B,Hq,d], LSE [B,Hq]) in float64.  Only the (b, kv-head) slices that the
    requested heads need are dequantised.
    """
    if kv_format not in ("int8", "fp8"):
        raise ValueError(kv_format)
    deq = dequant_int8_fp64 if kv_format == "int8" else dequant_fp8_fp64
    qf = _f64(q)
    B, Hq, d = qf.shape
    Hkv, L = k_codes.shape[1], k_codes.shape[2]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    lens = _as_list(seq_lens, B, L)
    W = 0 if k_recent is None else k_recent.shape[2]
    rlens = _as_list(recent_lens, B, W)
    work = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    by_kv = {}
    for b, h in work:
        by_kv.setdefault((b, h // G), []).append(h)

    def one(item):
        (b, kvh), hs = item
        n = lens[b]
        kk = deq(k_codes[b, kvh, :n], k_scales[b, kvh, :n])
        vv = deq(v_codes[b, kvh, :n], v_scales[b, kvh, :n])
        if W:
            r = rlens[b]
            kk = np.concatenate([kk, _f64(k_recent[b, kvh, :r])])
            vv = np.concatenate([vv, _f64(v_recent[b, kvh, :r])])
        qq = qf[b, hs][:, None, :]  # [g, 1, d]
        nv = np.array([kk.shape[0]])
        for j, h in enumerate(hs):
            oo, ll = _two_pass_rows(qq[j], kk, vv, tau, nv, 1)
            o[b, h], lse[b, h] = oo[0], ll[0]

    items = list(by_kv.items())
    nthreads = threads or _default_threads()
    if nthreads <= 1 or len(items) <= 1:
        for it in items:
            one(it)
    else:
        ctx = threadpool_limits(1) if threadpool_limits is not None else _Null()
        with ctx, ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one, items))
    return o, lse
