"""Seeded synthetic inputs for sparse attention.

This module only draws random tensors.  It contains none of the attention
arithmetic, so both the GPU path and the fp64 reference can consume its output
without sharing any of the computation.

Recipe (the operator pages give shapes, ranges and a call example, no dataset):
  * q, k ~ N(0, 1) drawn in fp32 from one CPU ``torch.Generator`` per call,
    then rounded (RNE) to the working dtype;
  * v is either the very same tensor as k (Dv == Dk), the prefix view
    ``k[..., :Dv]`` (the MLA latent-cache convention of the SparseFlashAttention
    page: value is the first Dv channels of key), or an independent N(0, 1)
    draw;
  * top-K indices: for every (b, s1, n2) group an independent uniform sample of
    topK distinct positions in [0, S2) -- the same law as ``randperm(S2)[:topK]``
    in the page's call example -- optionally sorted ascending;
  * BSR: every block row keeps its diagonal block plus a uniform sample, without
    replacement, of other column blocks; indices sorted ascending per row.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class SfaShape:
    """One top-K sparse attention problem (SparseFlashAttention page, sections 2-3)."""

    B: int
    S1: int
    S2: int
    N1: int
    N2: int
    Dk: int
    Dv: int
    topK: int
    dtype: str = "fp16"
    layout: str = "BSND"
    causal: bool = False
    scale: Optional[float] = None  # None -> 1/sqrt(Dk)
    value: str = "alias"  # "alias": v = k or k[..., :Dv]; "separate": independent draw
    sorted_indices: bool = False

    @property
    def G(self) -> int:
        return self.N1 // self.N2

    @property
    def scale_value(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.Dk)


@dataclasses.dataclass(frozen=True)
class BsrShape:
    """One block-sparse attention problem (flashinfer.sparse BlockSparseAttentionWrapper)."""

    M: int
    N: int
    R: int
    C: int
    Hq: int
    Hkv: int
    D: int
    blocks_per_row: int  # diagonal block + (blocks_per_row - 1) random others
    dtype: str = "fp16"
    causal: bool = False
    sm_scale: Optional[float] = None


@dataclasses.dataclass(frozen=True)
class VbsrShape:
    """One variable block-sparse problem (flashinfer.sparse VariableBlockSparseAttentionWrapper):
    every KV head cuts the M query rows and the N key rows into blocks whose sizes are drawn
    from `sizes` (the last block of a head takes the remainder; heads with fewer blocks are
    padded with empty ones), and each block row keeps its diagonal column block plus every
    other one with probability `density`."""

    M: int
    N: int
    Hq: int
    Hkv: int
    D: int
    sizes: tuple = (64, 128, 192)
    density: float = 0.25
    dtype: str = "fp16"
    causal: bool = False
    value: str = "separate"  # or "alias": v is k
    sm_scale: Optional[float] = None


# The five workloads: shapes inside the SparseFlashAttention support ranges and
# the BSR wrapper's example geometry scaled up.
WORKLOADS = {
    "tiny": SfaShape(B=1, S1=4, S2=64, N1=4, N2=1, Dk=64, Dv=64, topK=16, dtype="fp16",
                     layout="BSND", causal=False, scale=1.0 / 8.0),
    "gqa_decode": SfaShape(B=32, S1=1, S2=8192, N1=32, N2=8, Dk=128, Dv=128, topK=1024,
                           dtype="bf16", layout="BSND", causal=False),
    "mla_decode": SfaShape(B=16, S1=2, S2=8192, N1=128, N2=1, Dk=576, Dv=512, topK=2048,
                           dtype="bf16", layout="BNSD", causal=True, sorted_indices=True),
    "gqa_prefill": SfaShape(B=2, S1=1024, S2=4096, N1=64, N2=8, Dk=192, Dv=128, topK=512,
                            dtype="fp16", layout="BSND", causal=True),
    "bsr": BsrShape(M=8192, N=8192, R=64, C=64, Hq=32, Hkv=8, D=128, blocks_per_row=16,
                    dtype="fp16"),
}

# Variable block sizes at the BSR workload's scale: same sequence, heads and head dim, about the
# same density (14% of the attention matrix against 12.5%).
VBSR_WORKLOAD = VbsrShape(M=8192, N=8192, Hq=32, Hkv=8, D=128, sizes=(64, 128, 192), density=0.125, dtype="fp16")


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, dtype) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def sample_without_replacement(n_groups: int, S2: int, topK: int, g: torch.Generator,
                               sort: bool = False) -> torch.Tensor:
    """[n_groups, topK] int32; each row a uniform topK-subset of range(S2) in random order."""
    out = torch.empty((n_groups, topK), dtype=torch.int32)
    chunk = max(1, (1 << 24) // max(S2, 1))
    for a in range(0, n_groups, chunk):
        b = min(n_groups, a + chunk)
        keys = torch.rand((b - a, S2), generator=g)
        sel = torch.topk(keys, topK, dim=1).indices  # topK largest of iid uniforms
        if sort:
            sel, _ = torch.sort(sel, dim=1)
        out[a:b] = sel.to(torch.int32)
    return out


def sfa_inputs(shape: SfaShape, seed: int = 0):
    """Returns dict(q, k, v, idx) as CPU tensors in the shape's layout.

    BSND: q [B,S1,N1,Dk], k [B,S2,N2,Dk], v [B,S2,N2,Dv], idx [B,S1,N2,topK]
    BNSD: q [B,N1,S1,Dk], k [B,N2,S2,Dk], v [B,N2,S2,Dv], idx [B,N2,S1,topK]
    """
    s = shape
    dt = DTYPES[s.dtype]
    g = _gen(seed)
    if s.layout == "BSND":
        qshape, kshape, vshape = (s.B, s.S1, s.N1, s.Dk), (s.B, s.S2, s.N2, s.Dk), (s.B, s.S2, s.N2, s.Dv)
    elif s.layout == "BNSD":
        qshape, kshape, vshape = (s.B, s.N1, s.S1, s.Dk), (s.B, s.N2, s.S2, s.Dk), (s.B, s.N2, s.S2, s.Dv)
    else:
        raise ValueError(s.layout)
    q = _randn(qshape, g, dt)
    k = _randn(kshape, g, dt)
    if s.value == "alias":
        v = k if s.Dv == s.Dk else k[..., : s.Dv]
    else:
        v = _randn(vshape, g, dt)
    # groups are drawn in (b, s1, n2) order, then laid out per the layout
    idx = sample_without_replacement(s.B * s.S1 * s.N2, s.S2, s.topK, g, sort=s.sorted_indices)
    idx = idx.view(s.B, s.S1, s.N2, s.topK)
    if s.layout == "BNSD":
        idx = idx.permute(0, 2, 1, 3).contiguous()
    return {"q": q, "k": k, "v": v, "idx": idx}


def bsr_pattern(shape: BsrShape, g: torch.Generator):
    """indptr [MB+1], indices [nnz] int32: diagonal block + uniform others, sorted per row."""
    MB = (shape.M + shape.R - 1) // shape.R
    NB = shape.N // shape.C
    per_row = min(shape.blocks_per_row, NB)
    rows = []
    for br in range(MB):
        diag = min(br, NB - 1)
        others = [c for c in range(NB) if c != diag]
        if per_row - 1 > 0:
            pick = torch.randperm(len(others), generator=g)[: per_row - 1].tolist()
            chosen = sorted([diag] + [others[p] for p in pick])
        else:
            chosen = [diag]
        rows.append(chosen)
    indptr = torch.tensor([0] + [len(r) for r in rows], dtype=torch.int64).cumsum(0).to(torch.int32)
    indices = torch.tensor([c for r in rows for c in r], dtype=torch.int32)
    return indptr, indices


def bsr_inputs(shape: BsrShape, seed: int = 0):
    """Returns dict(q [M,Hq,D], k [N,Hkv,D], v [N,Hkv,D], indptr, indices) on the CPU."""
    s = shape
    dt = DTYPES[s.dtype]
    g = _gen(seed)
    q = _randn((s.M, s.Hq, s.D), g, dt)
    k = _randn((s.N, s.Hkv, s.D), g, dt)
    v = _randn((s.N, s.Hkv, s.D), g, dt)
    indptr, indices = bsr_pattern(s, g)
    return {"q": q, "k": k, "v": v, "indptr": indptr, "indices": indices}


def _cut(total: int, sizes, g: torch.Generator):
    out, acc = [], 0
    while acc < total:
        z = int(sizes[int(torch.randint(len(sizes), (1,), generator=g))])
        z = min(z, total - acc)
        out.append(z)
        acc += z
    return out


def vbsr_pattern(shape: VbsrShape, g: torch.Generator):
    """(block_mask_map [Hkv, MB, NB] bool, block_row_sz [Hkv, MB], block_col_sz [Hkv, NB] int32)."""
    s = shape
    rows = [_cut(s.M, s.sizes, g) for _ in range(s.Hkv)]
    cols = [_cut(s.N, s.sizes, g) for _ in range(s.Hkv)]
    MB = max(len(r) for r in rows)
    NB = max(len(c) for c in cols)
    rs = torch.zeros((s.Hkv, MB), dtype=torch.int32)
    cs = torch.zeros((s.Hkv, NB), dtype=torch.int32)
    bm = torch.zeros((s.Hkv, MB, NB), dtype=torch.bool)
    for h in range(s.Hkv):
        rs[h, : len(rows[h])] = torch.tensor(rows[h], dtype=torch.int32)
        cs[h, : len(cols[h])] = torch.tensor(cols[h], dtype=torch.int32)
        cstart = torch.cumsum(cs[h], 0) - cs[h]
        r0 = 0
        for i in range(len(rows[h])):
            keep = torch.rand((NB,), generator=g) < s.density
            # the diagonal block: the column block holding key position r0 * N / M
            pos = r0 * s.N // max(s.M, 1)
            diag = int(torch.searchsorted(cstart[: len(cols[h])], torch.tensor(pos), right=True)) - 1
            keep[max(diag, 0)] = True
            keep[len(cols[h]):] = False
            bm[h, i] = keep
            r0 += rows[h][i]
    return bm, rs, cs


def vbsr_inputs(shape: VbsrShape, seed: int = 0):
    """Returns dict(q [Hq, M, D], k [Hkv, N, D], v [Hkv, N, D] (v is k when aliased),
    block_mask_map, block_row_sz, block_col_sz) on the CPU (HND)."""
    s = shape
    dt = DTYPES[s.dtype]
    g = _gen(seed)
    q = _randn((s.Hq, s.M, s.D), g, dt)
    k = _randn((s.Hkv, s.N, s.D), g, dt)
    v = k if s.value == "alias" else _randn((s.Hkv, s.N, s.D), g, dt)
    bm, rs, cs = vbsr_pattern(s, g)
    return {"q": q, "k": k, "v": v, "block_mask_map": bm, "block_row_sz": rs, "block_col_sz": cs}


# FP8 inputs of the block-sparse run calls.  Recipe: the fp32 N(0,1) draws of the fp16
# workload, quantised per head the usual way: scale[h] = max |x[.., h, ..]| / (format
# maximum: 448 for E4M3, 57344 for E5M2), codes = x / scale[h] rounded by torch's float8
# conversion.  The attention then runs on codes * scale[h].
FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def fp8_quantise(x: torch.Tensor, fmt: str, head_axis: int):
    """(codes as a torch float8 tensor, fp32 scale per head) of an fp32 tensor."""
    red = [d for d in range(x.dim()) if d != head_axis]
    amax = x.abs().amax(dim=red).clamp_min(1e-12)
    scale = (amax / FP8_MAX[fmt]).to(torch.float32)
    shape = [1] * x.dim()
    shape[head_axis] = -1
    codes = (x / scale.reshape(shape)).to(FP8_TORCH[fmt])
    return codes, scale


def bsr_fp8_inputs(shape: BsrShape, q_fmt: str = "e4m3", kv_fmt: str = "e4m3", seed: int = 0):
    """FP8 form of bsr_inputs: dict(q, k, v codes (NHD), scale_q [Hq], scale_k, scale_v [Hkv],
    indptr, indices) on the CPU."""
    s = shape
    g = _gen(seed)
    q = torch.randn((s.M, s.Hq, s.D), generator=g, dtype=torch.float32)
    k = torch.randn((s.N, s.Hkv, s.D), generator=g, dtype=torch.float32)
    v = torch.randn((s.N, s.Hkv, s.D), generator=g, dtype=torch.float32)
    indptr, indices = bsr_pattern(s, g)
    q8, sq = fp8_quantise(q, q_fmt, 1)
    k8, sk = fp8_quantise(k, kv_fmt, 1)
    v8, sv = fp8_quantise(v, kv_fmt, 1)
    return {"q": q8, "k": k8, "v": v8, "scale_q": sq, "scale_k": sk, "scale_v": sv, "indptr": indptr,
            "indices": indices}
