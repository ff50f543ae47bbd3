"""fp64 CPU reference for sparse flash attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It is a plain scalar C statement of
the operator (``sfa_oracle.c``) behind a ctypes wrapper; it shares no code with
the GPU library and never runs on the product path.

Every function takes CPU tensors in the operator's own dtype (fp16/bf16 values
are widened exactly to fp64 here; FP8 codes are decoded from their bit fields by
``fp8_decode``) and returns fp64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

LAYOUTS = {"BSND": 0, "BNSD": 1}


def build(force: bool = True) -> str:
    """Compiles the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", _SRC, "-o", tmp, "-lpthread", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            L = ctypes.c_int64
            D = ctypes.c_double
            lib.oracle_sfa.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, D, P, L, P, P, I]
            lib.oracle_sfa.restype = I
            lib.oracle_dense_masked.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, P, L, P, P, I]
            lib.oracle_dense_masked.restype = I
            lib.oracle_bsr_mask.argtypes = [P, P, I, I, I, I, P]
            lib.oracle_bsr_mask.restype = I
            lib.oracle_bsr.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, D, P, L, P, P, I]
            lib.oracle_bsr.restype = I
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(t: torch.Tensor) -> torch.Tensor:
    """Exact widening to fp64, keeping the logical shape; the result is contiguous."""
    return t.detach().to("cpu").to(torch.float64).contiguous()


def _outer_strides(t: torch.Tensor):
    st = t.stride()
    if st[-1] != 1:
        raise ValueError("last dim must be contiguous")
    return (ctypes.c_int64 * 3)(*st[:3])


def _rows_arg(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data_as(ctypes.c_void_p), int(r.size)


def sfa(q, k, v, idx, scale: float, layout: str = "BSND", causal: bool = False,
        rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Top-K sparse attention (SparseFlashAttention page, section 2).

    Returns (y, lse): y [nrows, Dv] and lse [nrows] in fp64, one row per flat
    query id r = (b*S1 + s1)*N1 + n1 (all rows in that order when rows is None).
    """
    lib = _load()
    lay = LAYOUTS[layout]
    if lay == 0:
        B, S1, N1, Dk = q.shape
        S2, N2 = k.shape[1], k.shape[2]
    else:
        B, N1, S1, Dk = q.shape
        N2, S2 = k.shape[1], k.shape[2]
    Dv = v.shape[-1]
    topK = idx.shape[-1]
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    ix = idx.detach().to("cpu").to(torch.int32).contiguous()
    rr, rptr, nr = _rows_arg(rows)
    nrows = nr if rows is not None else B * S1 * N1
    y = np.zeros((nrows, Dv), dtype=np.float64)
    lse = np.zeros((nrows,), dtype=np.float64)
    rc = lib.oracle_sfa(qd.data_ptr(), _outer_strides(qd), kd.data_ptr(), _outer_strides(kd),
                        vd.data_ptr(), _outer_strides(vd), ix.data_ptr(), _outer_strides(ix),
                        B, S1, S2, N1, N2, Dk, Dv, topK, lay, int(bool(causal)), float(scale),
                        rptr, nr, y.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p),
                        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_sfa rejected the problem")
    return y, lse


def dense_masked(q, k, v, mask=None, causal: bool = False, scale: Optional[float] = None,
                 rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Dense attention with an optional boolean mask (single_prefill_with_kv_cache page).

    q [qo_len, Hq, Dqk], k [kv_len, Hkv, Dqk], v [kv_len, Hkv, Dvo]; mask [qo_len, kv_len]
    (True = attend) or None with causal = bottom-right causal.  Returns (y, lse) with
    y [nrows, Dvo] for flat ids r = qo_row*Hq + head.
    """
    lib = _load()
    qo_len, Hq, Dqk = q.shape
    kv_len, Hkv = k.shape[0], k.shape[1]
    Dvo = v.shape[-1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(Dqk))
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    mk = None
    if mask is not None:
        mk = torch.as_tensor(mask).to(torch.uint8).contiguous()
        assert tuple(mk.shape) == (qo_len, kv_len)
    rr, rptr, nr = _rows_arg(rows)
    nrows = nr if rows is not None else qo_len * Hq
    y = np.zeros((nrows, Dvo), dtype=np.float64)
    lse = np.zeros((nrows,), dtype=np.float64)
    rc = lib.oracle_dense_masked(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                 None if mk is None else mk.data_ptr(), int(bool(causal)),
                                 qo_len, kv_len, Hq, Hkv, Dqk, Dvo, float(scale), rptr, nr,
                                 y.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p),
                                 int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_dense_masked rejected the problem")
    return y, lse


def bsr_mask(indptr, indices, M: int, N: int, R: int, C: int) -> np.ndarray:
    """Dense [M, N] bool mask denoted by a BSR pattern (SciPy bsr_matrix semantics)."""
    lib = _load()
    ip = torch.as_tensor(indptr).to(torch.int32).contiguous()
    ix = torch.as_tensor(indices).to(torch.int32).contiguous()
    out = np.zeros((M, N), dtype=np.uint8)
    rc = lib.oracle_bsr_mask(ip.data_ptr(), ix.data_ptr(), M, N, R, C, out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("malformed BSR pattern")
    return out.astype(bool)


def bsr(q, k, v, indptr, indices, R: int, C: int, causal: bool = False, sm_scale: Optional[float] = None,
        rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None, mask=None):
    """Block-sparse attention (BlockSparseAttentionWrapper page).  q [M,Hq,D], k/v [N,Hkv,D].

    mask: optional per-block mask [nnz, R, C] (True = attend) of the plan page; with a mask
    the causal flag is ignored, as the page states.
    Returns (y, lse) with y [nrows, D] for flat ids r = row*Hq + head.
    """
    lib = _load()
    M, Hq, D = q.shape
    N, Hkv = k.shape[0], k.shape[1]
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    ip = torch.as_tensor(indptr).to(torch.int32).contiguous()
    ix = torch.as_tensor(indices).to(torch.int32).contiguous()
    rr, rptr, nr = _rows_arg(rows)
    nrows = nr if rows is not None else M * Hq
    y = np.zeros((nrows, D), dtype=np.float64)
    lse = np.zeros((nrows,), dtype=np.float64)
    bm = None if mask is None else torch.as_tensor(mask).to(torch.uint8).contiguous()
    if bm is not None and tuple(bm.shape) != (int(ip[-1]), R, C):
        raise ValueError("mask must be [nnz, R, C]")
    rc = lib.oracle_bsr(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ip.data_ptr(), ix.data_ptr(),
                        None if bm is None else bm.data_ptr(),
                        M, N, R, C, Hq, Hkv, D, int(bool(causal)), float(sm_scale or 0.0), rptr, nr,
                        y.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p),
                        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_bsr rejected the problem")
    return y, lse


def variable_block_mask(block_mask_map, block_row_sz, block_col_sz) -> np.ndarray:
    """Dense [Hkv, M, N] bool mask of a variable block pattern (VariableBlockSparseAttentionWrapper
    page, plan): KV head h cuts the rows into blocks of block_row_sz[h][i] rows and the columns
    into blocks of block_col_sz[h][j] columns, in order; every element of block (i, j) takes
    block_mask_map[h][i][j]."""
    bm = np.asarray(torch.as_tensor(block_mask_map).cpu(), dtype=bool)
    rs = np.asarray(torch.as_tensor(block_row_sz).cpu(), dtype=np.int64)
    cs = np.asarray(torch.as_tensor(block_col_sz).cpu(), dtype=np.int64)
    Hkv = bm.shape[0]
    masks = [np.repeat(np.repeat(bm[h], rs[h], axis=0), cs[h], axis=1) for h in range(Hkv)]
    if len({m.shape for m in masks}) != 1:
        raise ValueError("every KV head's block sizes must cover the same M x N")
    return np.stack(masks)


def vbsr(q, k, v, block_mask_map, block_row_sz, block_col_sz, causal: bool = False,
         sm_scale: Optional[float] = None, qrows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Variable block-sparse attention (VariableBlockSparseAttentionWrapper page): q [Hq, M, D],
    k / v [Hkv, N, D] (HND); query head n uses KV head n // (Hq / Hkv) and that head's mask,
    restricted by the bottom-right causal rule (key j <= row i + N - M) when causal.  Each KV
    head's query heads are one dense masked problem.  qrows: query rows to compute (all if None).
    Returns (y [Hq, R, Dv], lse [Hq, R]) in fp64, R = len(qrows) or M."""
    Hq, M, D = q.shape
    Hkv, N = k.shape[0], k.shape[1]
    Dv = v.shape[-1]
    G = Hq // Hkv
    mask = variable_block_mask(block_mask_map, block_row_sz, block_col_sz)
    if mask.shape[1:] != (M, N):
        raise ValueError("the block sizes do not cover q's and k's lengths")
    if causal:
        mask = mask & (np.arange(N)[None, None, :] <= np.arange(M)[None, :, None] + (N - M))
    scale = sm_scale if sm_scale else 1.0 / float(np.sqrt(D))
    rows_q = list(range(M)) if qrows is None else [int(r) for r in qrows]
    y = np.zeros((Hq, len(rows_q), Dv), dtype=np.float64)
    lse = np.zeros((Hq, len(rows_q)), dtype=np.float64)
    for h in range(Hkv):
        qg = q[h * G:(h + 1) * G].permute(1, 0, 2)  # [M, G, D]
        kg = k[h:h + 1].permute(1, 0, 2)            # [N, 1, D]
        vg = v[h:h + 1].permute(1, 0, 2)
        flat = None if qrows is None else [r * G + g for r in rows_q for g in range(G)]
        yh, lh = dense_masked(qg, kg, vg, mask=torch.from_numpy(mask[h]), causal=False, scale=scale, rows=flat,
                              nthreads=nthreads)
        y[h * G:(h + 1) * G] = yh.reshape(len(rows_q), G, Dv).transpose(1, 0, 2)
        lse[h * G:(h + 1) * G] = lh.reshape(len(rows_q), G).T
    return y, lse


# --- FP8 inputs of the block-sparse run calls -------------------------------------------
# The BlockSparseAttentionWrapper / VariableBlockSparseAttentionWrapper run sections take
# FP8 q, k, v with per-head dequantisation factors scale_q [num_qo_heads],
# scale_k / scale_v [num_kv_heads] (1.0 when absent); the operator page's precision table
# lists FLOAT8 E4M3 and E5M2.  The two encodings are those of the OCP 8-bit floating point
# specification: E4M3 (bias 7, no infinities, S.1111.111 is NaN) and E5M2 (bias 15, IEEE
# style: exponent 31 is inf / NaN).  A code's value here is computed from its bit fields.

FP8_FORMATS = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}


def fp8_decode(codes, fmt: str) -> np.ndarray:
    """fp64 value of every 8-bit code: sign, E exponent bits, M mantissa bits; exponent field
    0 is subnormal (m / 2^M) * 2^(1 - bias), otherwise (1 + m / 2^M) * 2^(e - bias)."""
    E, Mb, bias = FP8_FORMATS[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> Mb) & ((1 << E) - 1)
    m = (c & ((1 << Mb) - 1)).astype(np.float64)
    mag = np.where(e == 0, m / 2.0 ** Mb * 2.0 ** (1 - bias), (1.0 + m / 2.0 ** Mb) * np.exp2(e - bias))
    val = sign * mag
    if fmt == "e4m3":
        val = np.where((e == 15) & (m == 7), np.nan, val)
    else:
        val = np.where(e == 31, np.where(m == 0, sign * np.inf, np.nan), val)
    return val


def fp8_dequant(codes: torch.Tensor, fmt: str, scale=None, head_dim_axis: int = 1) -> torch.Tensor:
    """decode(codes) * scale[head] in fp64; codes is a uint8 (or float8) tensor and its axis
    head_dim_axis indexes the heads the scale vector runs over (None: scale 1)."""
    raw = codes.detach().cpu()
    if raw.dtype != torch.uint8:
        raw = raw.view(torch.uint8)
    val = fp8_decode(raw.numpy(), fmt)
    if scale is not None:
        s = np.asarray(torch.as_tensor(scale).detach().cpu().to(torch.float64))
        shape = [1] * val.ndim
        shape[head_dim_axis] = -1
        val = val * s.reshape(shape)
    return torch.from_numpy(np.ascontiguousarray(val))


def bsr_fp8(q8, k8, v8, q_fmt: str, kv_fmt: str, scale_q, scale_k, scale_v, indptr, indices, R: int, C: int,
            causal: bool = False, sm_scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
            nthreads: Optional[int] = None, mask=None):
    """Block-sparse attention of FP8 q [M,Hq,D], k / v [N,Hkv,D] (NHD codes) with per-head
    factors: the BSR attention of q * scale_q[h], k * scale_k[hk], v * scale_v[hk], in fp64."""
    qd = fp8_dequant(q8, q_fmt, scale_q, 1)
    kd = fp8_dequant(k8, kv_fmt, scale_k, 1)
    vd = fp8_dequant(v8, kv_fmt, scale_v, 1)
    return bsr(qd, kd, vd, indptr, indices, R, C, causal=causal, sm_scale=sm_scale, rows=rows,
               nthreads=nthreads, mask=mask)


def vbsr_fp8(q8, k8, v8, q_fmt: str, kv_fmt: str, scale_q, scale_k, scale_v, block_mask_map, block_row_sz,
             block_col_sz, causal: bool = False, sm_scale: Optional[float] = None,
             qrows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Variable block-sparse attention of FP8 q [Hq,M,D], k / v [Hkv,N,D] (HND codes) with
    per-head factors, in fp64."""
    qd = fp8_dequant(q8, q_fmt, scale_q, 0)
    kd = fp8_dequant(k8, kv_fmt, scale_k, 0)
    vd = fp8_dequant(v8, kv_fmt, scale_v, 0)
    return vbsr(qd, kd, vd, block_mask_map, block_row_sz, block_col_sz, causal=causal, sm_scale=sm_scale,
                qrows=qrows, nthreads=nthreads)


def index_report(idx, S2: int, layout: str = "BSND") -> dict:
    """The operator page's index rule (section 3: every sparseIndices value lies in [0, S2)),
    checked row by row: slots outside the range, and index rows (b, s1, n2) that list some
    position more than once."""
    a = np.asarray(torch.as_tensor(idx).cpu(), dtype=np.int64)
    if layout == "BNSD":
        a = a.transpose(0, 2, 1, 3)
    rows = a.reshape(-1, a.shape[-1])
    oob = int(((rows < 0) | (rows >= S2)).sum())
    dup = 0
    for r in rows:
        ok = r[(r >= 0) & (r < S2)]
        if len(np.unique(ok)) != len(ok):
            dup += 1
    return {"out_of_range": oob, "duplicate_rows": dup}
