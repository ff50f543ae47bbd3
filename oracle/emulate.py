"""Numerics emulator for the top-K sparse attention: the definition of the operator page
(section 2) evaluated with the roundings a GPU kernel of this form applies, to decide at
which precision the softmax weights P may enter the P V product.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: it is used by the tests to show which
P precision meets the page's precision standard (section 4); it shares no code with the GPU
library.

Rounding points emulated, in order:
  * logits s = q . k accumulated in fp32 (products of fp16 / bf16 values are exact in fp32);
  * online softmax over chunks of `chunk` slots in fp32: running max m, P = exp(s * scale - m),
    running sum l, accumulator rescale by exp(m_old - m_new) when the max moves;
  * P rounded for the product with V: "single" (P rounded once to the input dtype), "hilo"
    (P as hi = round(P) plus lo = round(P - hi), both in the input dtype) or "fp32";
  * P V accumulated in fp32; y = acc / l rounded to the input dtype (nearest even).
Masked slots (causal rule of section 2) get P = 0; a row with no unmasked slot gives 0.
"""
from __future__ import annotations

import numpy as np
import torch


def _round16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to fp16 / bf16 (nearest even), returned as fp32."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000  # nearest even on the upper 16 bits
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


def p_for_pv(p: np.ndarray, p_mode: str, dtype: str) -> np.ndarray:
    """The value P takes in the P V product (fp32 array): "single" rounds it once to the 16-bit
    input type; "hilo" is hi + lo with hi = round(P) and lo = round(P - hi), the two 16-bit
    operands the kernels multiply V by (P - hi is exact in fp32); "fp32" keeps P."""
    p = np.asarray(p, dtype=np.float32)
    if p_mode == "single":
        return _round16(p, dtype)
    if p_mode == "hilo":
        hi = _round16(p, dtype)
        return hi + _round16(p - hi, dtype)
    if p_mode == "fp32":
        return p
    raise ValueError(p_mode)


def topk_attention(q, k, v, idx, scale: float, layout: str, causal: bool, p_mode: str, dtype: str,
                   rows=None, chunk: int = 32, round_output: bool = True) -> np.ndarray:
    """Emulated y [len(rows), Dv] (fp32 values of the output dtype; the fp32 quotient before
    that rounding with round_output=False) for flat rows r = ((b * S1 + s1) * N1 + n1) (all
    rows when None)."""
    if layout == "BNSD":
        q, k, v, idx = (t.permute(0, 2, 1, 3) for t in (q, k, v, idx))
    q = q.float().numpy()
    k = k.float().numpy()
    v = v.float().numpy()
    idx = idx.numpy().astype(np.int64)
    B, S1, N1, Dk = q.shape
    S2, N2, Dv = k.shape[1], k.shape[2], v.shape[-1]
    G = N1 // N2
    topK = idx.shape[-1]
    rows = np.arange(B * S1 * N1) if rows is None else np.asarray(rows)
    b, rem = rows // (S1 * N1), rows % (S1 * N1)
    s1, n1 = rem // N1, rem % N1
    n2 = n1 // G
    sel = idx[b, s1, n2]                                     # [R, topK]
    ks = k[b[:, None], sel, n2[:, None]]                     # [R, topK, Dk]
    vs = v[b[:, None], sel, n2[:, None]]                     # [R, topK, Dv]
    qs = q[b, s1, n1]                                        # [R, Dk]
    s = np.einsum("rd,rtd->rt", qs.astype(np.float64), ks.astype(np.float64)).astype(np.float32)
    valid = np.ones_like(sel, dtype=bool)
    if causal:
        valid = sel <= (s1 + (S2 - S1))[:, None]
    R = len(rows)
    m = np.full(R, -np.inf, dtype=np.float32)
    lsum = np.zeros(R, dtype=np.float32)
    acc = np.zeros((R, Dv), dtype=np.float32)
    sc = np.float32(scale)
    for c0 in range(0, topK, chunk):
        sl = slice(c0, min(topK, c0 + chunk))
        x = np.where(valid[:, sl], s[:, sl] * sc, np.float32(-np.inf)).astype(np.float32)
        cmax = x.max(axis=1)
        m_new = np.maximum(m, cmax)
        m_use = np.where(np.isfinite(m_new), m_new, np.float32(0))
        alpha = np.where(np.isfinite(m), np.exp(m - m_use), np.float32(0)).astype(np.float32)
        p = np.exp(x - m_use[:, None]).astype(np.float32)  # exp(-inf) = 0 for masked slots
        lsum = lsum * alpha + p.sum(axis=1, dtype=np.float32)
        pq = p_for_pv(p, p_mode, dtype)
        acc = acc * alpha[:, None] + np.einsum("rt,rtd->rd", pq, vs[:, sl]).astype(np.float32)
        m = m_new
    inv = np.where(lsum > 0, np.float32(1) / np.where(lsum > 0, lsum, 1), np.float32(0))
    y = (acc * inv[:, None]).astype(np.float32)
    return _round16(y, dtype) if round_output else y
