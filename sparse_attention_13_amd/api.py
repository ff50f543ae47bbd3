"""PyTorch-facing calls.  They allocate outputs with torch, read pointers, strides and
the current HIP stream, and call libsfa through ``binding``; every step of the
attention runs in the HIP kernels.

* ``sparse_flash_attention`` -- the SparseFlashAttention operator's interface
  (query, key, value, sparseIndices, scaleValue, inputLayout, is_causal) -> y,
  optionally also returning the log-sum-exp.
* ``BlockSparseAttentionWrapper`` -- plan(indptr, indices, M, N, R, C,
  num_qo_heads, num_kv_heads, head_dim, ...) once, then run(q, k, v).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import binding

_TORCH_DTYPES = {torch.float16: "fp16", torch.bfloat16: "bf16"}
_FP8_DTYPES = {torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2"}


def _compute_dtype(q_data_type, o_data_type):
    """dtype the plan computes and outputs in: the q dtype, or for FP8 inputs the output
    dtype (the plan page's o_data_type, half by default; only fp16 is supported)."""
    if q_data_type in _FP8_DTYPES:
        o = o_data_type if o_data_type is not None else torch.float16
        if o != torch.float16:
            raise binding.SfaError("plan", 2)
        return o
    if q_data_type not in _TORCH_DTYPES or (o_data_type is not None and o_data_type != q_data_type):
        raise binding.SfaError("plan", 2)
    return q_data_type


def _fp8_scales(scales, counts, device):
    """Device fp32 [heads] pointers of scale_q / scale_k / scale_v (None: factor 1)."""
    keep, ptrs = [], []
    for s, n in zip(scales, counts):
        if s is None:
            ptrs.append(None)
            continue
        t = torch.as_tensor(s, dtype=torch.float32, device=device).reshape(-1).contiguous()
        if t.numel() != n:
            raise ValueError(f"a scale tensor must hold one factor per head ({n})")
        keep.append(t)
        ptrs.append(t.data_ptr())
    return keep, ptrs


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int):
    if rc != binding.SFA_OK:
        raise binding.SfaError(fn, rc)


def _dtype_name(t: torch.Tensor) -> str:
    if t.dtype not in _TORCH_DTYPES:
        raise binding.SfaError("sparse_flash_attention", 2)
    return _TORCH_DTYPES[t.dtype]


def sfa_shape_of(query, key, value, sparseIndices, inputLayout="BSND"):
    """Problem sizes of one call, after checking that the four tensors agree with each other
    (SparseFlashAttention operator page, section 3: key (B,S2,N2,Dk), value (B,S2,N2,Dv) and
    sparseIndices (B,S1,N2,topK) in BSND; BNSD swaps the S and N dims)."""
    if inputLayout not in ("BSND", "BNSD"):
        raise binding.SfaError("sparse_flash_attention", 3)
    for name, t in (("query", query), ("key", key), ("value", value), ("sparseIndices", sparseIndices)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be a 4-d tensor ({inputLayout})")
    if inputLayout == "BSND":
        B, S1, N1, Dk = query.shape
        S2, N2 = key.shape[1], key.shape[2]
        want_k = (B, S2, N2, Dk)
        want_v = (B, S2, N2, value.shape[-1])
        want_i = (B, S1, N2, sparseIndices.shape[-1])
    else:
        B, N1, S1, Dk = query.shape
        N2, S2 = key.shape[1], key.shape[2]
        want_k = (B, N2, S2, Dk)
        want_v = (B, N2, S2, value.shape[-1])
        want_i = (B, N2, S1, sparseIndices.shape[-1])
    for name, t, want in (("key", key, want_k), ("value", value, want_v), ("sparseIndices", sparseIndices, want_i)):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}; {inputLayout} with query {tuple(query.shape)} "
                             f"and key {tuple(key.shape)} needs {want}")
    return binding.make_shape(B, S1, S2, N1, N2, Dk, value.shape[-1], sparseIndices.shape[-1])


def _check_device_tensor(name: str, t: torch.Tensor, device: torch.device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def workspace_bytes(query, key, value, sparseIndices, inputLayout="BSND", is_causal=False) -> int:
    shape = sfa_shape_of(query, key, value, sparseIndices, inputLayout)
    return binding.sfa_workspace_bytes(shape, binding.DTYPE[_dtype_name(query)], int(bool(is_causal)))


def sparse_flash_attention(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                           sparseIndices: torch.Tensor, scaleValue: float, inputLayout: str = "BSND",
                           is_causal: bool = False, *, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                           workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """y = softmax(Q K_sel^T * scaleValue [causal]) V_sel over the topK selected rows.

    Shapes (BSND): query [B,S1,N1,Dk], key [B,S2,N2,Dk], value [B,S2,N2,Dv] (may be
    ``key[..., :Dv]``), sparseIndices int32 [B,S1,N2,topK]; BNSD swaps the S and N dims.
    Returns y [B,S1,N1,Dv] (BSND) / [B,N1,S1,Dv] (BNSD), or (y, lse) with ``return_lse``.
    With ``prepare=True`` nothing is launched: a PreparedCall that runs this exact call is returned.
    """
    lib = binding.load()
    del lib
    dt = _dtype_name(query)
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise binding.SfaError("sparse_flash_attention", 2)
    if sparseIndices.dtype != torch.int32:
        raise TypeError("sparseIndices must be int32")
    # shapes first (host-only checks), then devices: nothing is launched on a mismatch
    shape = sfa_shape_of(query, key, value, sparseIndices, inputLayout)
    for t in (query, key, value, sparseIndices):
        if t.stride(-1) != 1:
            raise binding.SfaError("sparse_flash_attention", 3)
    if not query.is_cuda:
        raise ValueError("sparse_flash_attention runs on the GPU: pass device tensors")
    dev = query.device
    for name, t in (("key", key), ("value", value), ("sparseIndices", sparseIndices)):
        _check_device_tensor(name, t, dev)
    if out is not None:
        _check_device_tensor("out", out, dev)
        if out.dtype != query.dtype:
            raise ValueError(f"out must have the query dtype {query.dtype} (got {out.dtype})")
    if lse is not None:
        _check_device_tensor("lse", lse, dev)
    if workspace is not None:
        _check_device_tensor("workspace", workspace, dev)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    if inputLayout == "BSND":
        oshape = (shape.B, shape.S1, shape.N1, shape.Dv)
        lshape = (shape.B, shape.S1, shape.N1)
    else:
        oshape = (shape.B, shape.N1, shape.S1, shape.Dv)
        lshape = (shape.B, shape.N1, shape.S1)
    if out is None:
        out = torch.empty(oshape, dtype=query.dtype, device=query.device)
    if (return_lse or lse is not None) and lse is None:
        lse = torch.empty(lshape, dtype=torch.float32, device=query.device)
    if lse is not None and (tuple(lse.shape) != lshape or not lse.is_contiguous() or lse.dtype != torch.float32):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {lshape}")
    if tuple(out.shape) != oshape or out.stride(-1) != 1:
        raise ValueError(f"out must have shape {oshape} with a contiguous last dim")
    strides = binding.make_strides(query.stride(), key.stride(), value.stride(), sparseIndices.stride(),
                                   out.stride())
    need = binding.sfa_workspace_bytes(shape, binding.DTYPE[dt], int(bool(is_causal)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (shape, strides, binding.DTYPE[dt], binding.LAYOUT[inputLayout], int(bool(is_causal)),
            float(scaleValue), query.data_ptr(), key.data_ptr(), value.data_ptr(), sparseIndices.data_ptr(),
            out.data_ptr(), lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes)
    if prepare:
        keep = (query, key, value, sparseIndices, out, lse, workspace, shape, strides)
        fn, raw = binding.sfa_run_prepared(*args)
        return PreparedCall("sfa_run", fn, raw, keep, (out, lse) if return_lse else out)
    rc = binding.sfa_run(*args, _stream_handle())
    _check("sfa_run", rc)
    return (out, lse) if return_lse else out


def validate_indices(sparseIndices: torch.Tensor, S2: int, inputLayout: str = "BSND") -> dict:
    """Debug check of sparseIndices [B,S1,N2,topK] (BSND) / [B,N2,S1,topK] (BNSD) on the GPU:
    {"out_of_range": slots outside [0, S2), "duplicate_rows": rows listing a position twice}.
    Synchronises the current stream."""
    if sparseIndices.dtype != torch.int32 or not sparseIndices.is_cuda or sparseIndices.dim() != 4 \
            or sparseIndices.stride(-1) != 1:
        raise ValueError("sparseIndices must be a 4-d int32 device tensor with a contiguous last dim")
    if inputLayout == "BSND":
        B, S1, N2, topK = sparseIndices.shape
    elif inputLayout == "BNSD":
        B, N2, S1, topK = sparseIndices.shape
    else:
        raise binding.SfaError("sfa_validate_indices", 3)
    shape = binding.make_shape(B, S1, S2, N2, N2, 64, 64, topK)
    st = sparseIndices.stride()
    strides = binding.make_strides((0, 0, 0), (0, 0, 0), (0, 0, 0), st[:3], (0, 0, 0))
    counts = torch.empty(2, dtype=torch.int32, device=sparseIndices.device)
    rc = binding.sfa_validate_indices(shape, strides, binding.LAYOUT[inputLayout], sparseIndices.data_ptr(),
                                      counts.data_ptr(), _stream_handle())
    _check("sfa_validate_indices", rc)
    c = counts.cpu().tolist()
    return {"out_of_range": int(c[0]), "duplicate_rows": int(c[1])}


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


class _PlanBuffers:
    """Device memory of a block-sparse plan, as the flashinfer.sparse page splits it: the
    caller's float workspace (constructor / reset_workspace_buffer) receives the split-k
    partial results of every run; the int workspace keeps the plan's expanded key lists.
    A buffer the caller gave is used as it is and must be large enough (else SfaError with
    SFA_ERR_WORKSPACE); without one, the wrapper allocates its own."""

    def __init__(self, float_ws: Optional[torch.Tensor]):
        self.float_ws, self.float_user = float_ws, float_ws is not None
        self.int_ws, self.int_user = None, False
        self._check_user(float_ws, "float_workspace_buffer")

    @staticmethod
    def _check_user(t, name):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")

    def reset(self, float_ws: torch.Tensor, int_ws: Optional[torch.Tensor]):
        self._check_user(float_ws, "float_workspace_buffer")
        self._check_user(int_ws, "int_workspace_buffer")
        self.float_ws, self.float_user = float_ws, float_ws is not None
        if int_ws is not None:
            self.int_ws, self.int_user = int_ws, True

    def ensure(self, fn: str, need_int: int, need_float: int, device):
        if self.int_user:
            if _nbytes(self.int_ws) < need_int:
                raise binding.SfaError(fn, 10)
        elif self.int_ws is None or _nbytes(self.int_ws) < need_int:
            self.int_ws = torch.empty(max(need_int, 16), dtype=torch.uint8, device=device)
        if self.float_user:
            if _nbytes(self.float_ws) < need_float:
                raise binding.SfaError(fn, 10)
        elif need_float > 0 and (self.float_ws is None or _nbytes(self.float_ws) < need_float):
            self.float_ws = torch.empty(need_float, dtype=torch.uint8, device=device)

    def args(self):
        f = self.float_ws
        return (self.int_ws.data_ptr(), _nbytes(self.int_ws), f.data_ptr() if f is not None else None,
                _nbytes(f) if f is not None else 0)


def _check_lse(fn: str, lse: Optional[torch.Tensor], shape, device):
    """lse given by the caller: fp32, contiguous, the output's row x head shape, on the device."""
    if lse is None:
        return
    if tuple(lse.shape) != tuple(shape) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError(f"{fn}: lse must be a contiguous float32 tensor of shape {tuple(shape)}")
    _check_device_tensor("lse", lse, device)


class PreparedCall:
    """A library call with every argument marshalled once; calling it enqueues the kernels on
    the current stream with a single foreign call (for loops that launch the same problem)."""

    def __init__(self, name, fn, args, keepalive, result):
        self.name, self.fn, self.args, self.keepalive, self.result = name, fn, args, keepalive, result

    def __call__(self, stream: Optional[int] = None):
        rc = self.fn(*self.args, ctypes.c_void_p(_stream_handle() if stream is None else stream))
        if rc != binding.SFA_OK:
            raise binding.SfaError(self.name, rc)
        return self.result


class BlockSparseAttentionWrapper:
    """Block-sparse attention with a BSR mask (flashinfer.sparse page): plan once, run many times."""

    def __init__(self, float_workspace_buffer: Optional[torch.Tensor] = None, backend: str = "auto"):
        """float_workspace_buffer: device scratch for the split-k partial results of run()
        (the page recommends 128 MB); when omitted the wrapper allocates what its plans need.
        backend is accepted for the page's signature; there is one implementation."""
        self._bufs = _PlanBuffers(float_workspace_buffer)
        self._fp8_ws = None
        self._plan = None
        self._meta = None

    def reset_workspace_buffer(self, float_workspace_buffer: torch.Tensor,
                               int_workspace_buffer: Optional[torch.Tensor] = None):
        """Takes effect at the next plan(), which places its data in these buffers."""
        self._bufs.reset(float_workspace_buffer, int_workspace_buffer)

    def plan(self, indptr, indices, M: int, N: int, R: int, C: int, num_qo_heads: int, num_kv_heads: int,
             head_dim: int, mask: Optional[torch.Tensor] = None, causal: bool = False,
             sm_scale: Optional[float] = None, q_data_type=torch.float16, kv_data_type=None, o_data_type=None,
             device=None):
        """mask: optional [nnz, R, C] boolean per-block mask (True = attend); with a mask the
        causal flag is ignored, as the plan page states.  q_data_type / kv_data_type may be
        torch.float8_e4m3fn or torch.float8_e5m2 (run() then takes scale_q / scale_k /
        scale_v); the output is then o_data_type, fp16."""
        binding.load()
        ip = torch.as_tensor(indptr).to("cpu", torch.int32).contiguous()
        ix = torch.as_tensor(indices).to("cpu", torch.int32).contiguous()
        bm = None
        if mask is not None:
            bm = torch.as_tensor(mask).to("cpu", torch.uint8).contiguous()
            if tuple(bm.shape) != (int(ip[-1]) if ip.numel() else 0, R, C):
                raise ValueError("mask must have shape (nnz, R, C)")
        bm_ptr = bm.data_ptr() if bm is not None and bm.numel() else None
        if device is None:
            device = torch.device("cuda", torch.cuda.current_device())
        ix_ptr = ix.data_ptr() if ix.numel() else None
        need = binding.bsr_plan_workspace_bytes(ip.data_ptr(), ix_ptr, M, N, R, C, num_qo_heads, num_kv_heads,
                                                head_dim, bm_ptr)
        need_f = binding.bsr_plan_float_workspace_bytes(ip.data_ptr(), ix_ptr, M, N, R, C, num_qo_heads,
                                                        num_kv_heads, head_dim)
        self._bufs.ensure("bsr_plan", need, need_f, device)
        if self._plan is not None:
            binding.bsr_destroy(self._plan)
            self._plan = None
        odt = _compute_dtype(q_data_type, o_data_type)
        kvdt = kv_data_type if kv_data_type is not None else q_data_type
        if (q_data_type in _FP8_DTYPES) != (kvdt in _FP8_DTYPES):
            raise binding.SfaError("bsr_plan", 2)
        dt = _TORCH_DTYPES[odt]
        iw, iwb, fw, fwb = self._bufs.args()
        rc, handle = binding.bsr_plan(ip.data_ptr(), ix.data_ptr(), M, N, R, C, num_qo_heads, num_kv_heads,
                                      head_dim, int(bool(causal)), float(sm_scale or 0.0), binding.DTYPE[dt],
                                      iw, iwb, _stream_handle(), bm_ptr, fw, fwb)
        _check("bsr_plan", rc)
        self._plan = handle
        self._meta = dict(M=M, N=N, Hq=num_qo_heads, Hkv=num_kv_heads, D=head_dim, dtype=q_data_type,
                          kv_dtype=kvdt, o_dtype=odt)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale_q=None, scale_k=None, scale_v=None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, return_lse: bool = False):
        """scale_q [Hq], scale_k / scale_v [Hkv]: per-head factors of FP8 inputs (1.0 if None)."""
        if self._plan is None:
            raise binding.SfaError("bsr_run", 11)
        m = self._meta
        if out is None:
            out = torch.empty((m["M"], m["Hq"], m["D"]), dtype=m["o_dtype"], device=q.device)
        if (return_lse or lse is not None) and lse is None:
            lse = torch.empty((m["M"], m["Hq"]), dtype=torch.float32, device=q.device)
        for t in (q, k, v, out):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("q, k, v and out must be contiguous device tensors (NHD)")
        if q.dtype != m["dtype"] or k.dtype != m["kv_dtype"] or v.dtype != k.dtype or out.dtype != m["o_dtype"]:
            raise binding.SfaError("bsr_run", 2)
        if tuple(q.shape) != (m["M"], m["Hq"], m["D"]) or tuple(k.shape) != (m["N"], m["Hkv"], m["D"]) \
                or tuple(v.shape) != (m["N"], m["Hkv"], m["D"]) or tuple(out.shape) != tuple(q.shape):
            raise binding.SfaError("bsr_run", 4)
        for name, t in (("k", k), ("v", v), ("out", out)):
            _check_device_tensor(name, t, q.device)
        _check_lse("bsr_run", lse, (m["M"], m["Hq"]), q.device)
        lse_ptr = lse.data_ptr() if lse is not None else None
        if q.dtype in _FP8_DTYPES:
            keep, (sq, sk, sv) = _fp8_scales((scale_q, scale_k, scale_v), (m["Hq"], m["Hkv"], m["Hkv"]), q.device)
            if scale_v is scale_k:
                sv = sk
            need = binding.bsr_fp8_workspace_bytes(self._plan)
            if self._fp8_ws is None or self._fp8_ws.numel() < need:
                self._fp8_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            rc = binding.bsr_run_fp8(self._plan, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     binding.FP8[_FP8_DTYPES[q.dtype]], binding.FP8[_FP8_DTYPES[k.dtype]], sq, sk, sv,
                                     out.data_ptr(), lse_ptr, self._fp8_ws.data_ptr(), self._fp8_ws.numel(),
                                     _stream_handle())
            del keep
        else:
            rc = binding.bsr_run(self._plan, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                 _stream_handle())
        _check("bsr_run", rc)
        return (out, lse) if return_lse else out

    def __del__(self):
        try:
            if self._plan is not None:
                binding.bsr_destroy(self._plan)
        except Exception:
            pass


class VariableBlockSparseAttentionWrapper:
    """Block-sparse attention with variable block sizes and a block pattern per KV head
    (flashinfer.sparse page, VariableBlockSparseAttentionWrapper): plan once, run many times.
    q [Hq, M, D], k / v [Hkv, N, D] (HND); the output follows q's layout, [Hq, M, D], and the
    LSE is [Hq, M]."""

    def __init__(self, float_workspace_buffer: Optional[torch.Tensor] = None, backend: str = "auto"):
        """float_workspace_buffer: device scratch for the split-k partial results (as for
        BlockSparseAttentionWrapper); backend is accepted for the page's signature."""
        self._bufs = _PlanBuffers(float_workspace_buffer)
        self._fp8_ws = None
        self._plan = None
        self._meta = None

    def reset_workspace_buffer(self, float_workspace_buffer: torch.Tensor,
                               int_workspace_buffer: Optional[torch.Tensor] = None):
        """Takes effect at the next plan()."""
        self._bufs.reset(float_workspace_buffer, int_workspace_buffer)

    def plan(self, block_mask_map, block_row_sz, block_col_sz, num_qo_heads: int, num_kv_heads: int,
             head_dim: int, causal: bool = False, sm_scale: Optional[float] = None, q_data_type=torch.float16,
             kv_data_type=None, o_data_type=None, device=None):
        """block_mask_map (Hkv, MB, NB) bool, block_row_sz (Hkv, MB) and block_col_sz (Hkv, NB)
        int32; every KV head's row sizes sum to the query length, its column sizes to the key
        length."""
        binding.load()
        bm = torch.as_tensor(block_mask_map).to("cpu", torch.uint8).contiguous()
        rs = torch.as_tensor(block_row_sz).to("cpu", torch.int32).contiguous()
        cs = torch.as_tensor(block_col_sz).to("cpu", torch.int32).contiguous()
        if bm.dim() != 3 or bm.shape[0] != num_kv_heads:
            raise ValueError("block_mask_map must have shape (num_kv_heads, MB, NB)")
        Hkv, MB, NB = (int(x) for x in bm.shape)
        if tuple(rs.shape) != (Hkv, MB) or tuple(cs.shape) != (Hkv, NB):
            raise ValueError("block_row_sz must be (num_kv_heads, MB) and block_col_sz (num_kv_heads, NB)")
        if device is None:
            device = torch.device("cuda", torch.cuda.current_device())
        ptrs = (bm.data_ptr() if bm.numel() else None, rs.data_ptr() if rs.numel() else None,
                cs.data_ptr() if cs.numel() else None)
        need = binding.vbsr_plan_workspace_bytes(*ptrs, Hkv, MB, NB, num_qo_heads, head_dim)
        need_f = binding.vbsr_plan_float_workspace_bytes(*ptrs, Hkv, MB, NB, num_qo_heads, head_dim)
        self._bufs.ensure("vbsr_plan", need, need_f, device)
        if self._plan is not None:
            binding.vbsr_destroy(self._plan)
            self._plan = None
        odt = _compute_dtype(q_data_type, o_data_type)
        kvdt = kv_data_type if kv_data_type is not None else q_data_type
        if (q_data_type in _FP8_DTYPES) != (kvdt in _FP8_DTYPES):
            raise binding.SfaError("vbsr_plan", 2)
        dt = _TORCH_DTYPES[odt]
        iw, iwb, fw, fwb = self._bufs.args()
        rc, handle = binding.vbsr_plan(*ptrs, Hkv, MB, NB, num_qo_heads, head_dim, int(bool(causal)),
                                       float(sm_scale or 0.0), binding.DTYPE[dt], iw, iwb, _stream_handle(), fw, fwb)
        _check("vbsr_plan", rc)
        self._plan = handle
        M = int(rs[0].sum()) if MB else 0
        N = int(cs[0].sum())
        self._meta = dict(M=M, N=N, Hq=num_qo_heads, Hkv=Hkv, D=head_dim, dtype=q_data_type, kv_dtype=kvdt,
                          o_dtype=odt)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale_q=None, scale_k=None, scale_v=None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, return_lse: bool = False):
        """scale_q [Hq], scale_k / scale_v [Hkv]: per-head factors of FP8 inputs (1.0 if None)."""
        if self._plan is None:
            raise binding.SfaError("vbsr_run", 11)
        m = self._meta
        if out is None:
            out = torch.empty((m["Hq"], m["M"], m["D"]), dtype=m["o_dtype"], device=q.device)
        if (return_lse or lse is not None) and lse is None:
            lse = torch.empty((m["Hq"], m["M"]), dtype=torch.float32, device=q.device)
        for t in (q, k, v, out):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("q, k, v and out must be contiguous device tensors (HND)")
        if q.dtype != m["dtype"] or k.dtype != m["kv_dtype"] or v.dtype != k.dtype or out.dtype != m["o_dtype"]:
            raise binding.SfaError("vbsr_run", 2)
        if tuple(q.shape) != (m["Hq"], m["M"], m["D"]) or tuple(k.shape) != (m["Hkv"], m["N"], m["D"]) \
                or tuple(v.shape) != (m["Hkv"], m["N"], m["D"]) or tuple(out.shape) != tuple(q.shape) \
                or (lse is not None and (tuple(lse.shape) != (m["Hq"], m["M"]) or lse.dtype != torch.float32
                                         or not lse.is_contiguous())):
            raise binding.SfaError("vbsr_run", 4)
        for name, t in (("k", k), ("v", v), ("out", out)):
            _check_device_tensor(name, t, q.device)
        _check_lse("vbsr_run", lse, (m["Hq"], m["M"]), q.device)
        lse_ptr = lse.data_ptr() if lse is not None else None
        if q.dtype in _FP8_DTYPES:
            keep, (sq, sk, sv) = _fp8_scales((scale_q, scale_k, scale_v), (m["Hq"], m["Hkv"], m["Hkv"]), q.device)
            if scale_v is scale_k:
                sv = sk
            need = binding.vbsr_fp8_workspace_bytes(self._plan)
            if self._fp8_ws is None or self._fp8_ws.numel() < need:
                self._fp8_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            rc = binding.vbsr_run_fp8(self._plan, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      binding.FP8[_FP8_DTYPES[q.dtype]], binding.FP8[_FP8_DTYPES[k.dtype]], sq, sk,
                                      sv, out.data_ptr(), lse_ptr, self._fp8_ws.data_ptr(), self._fp8_ws.numel(),
                                      _stream_handle())
            del keep
        else:
            rc = binding.vbsr_run(self._plan, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                  _stream_handle())
        _check("vbsr_run", rc)
        return (out, lse) if return_lse else out

    def __del__(self):
        try:
            if self._plan is not None:
                binding.vbsr_destroy(self._plan)
        except Exception:
            pass


def single_prefill_with_kv_cache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 custom_mask: Optional[torch.Tensor] = None, causal: bool = False,
                                 kv_layout: str = "NHD", sm_scale: Optional[float] = None, return_lse: bool = False,
                                 *, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None):
    """Dense attention of one request (flashinfer.prefill.single_prefill_with_kv_cache page).

    q [qo_len, Hq, Dqk]; k [kv_len, Hkv, Dqk] and v [kv_len, Hkv, Dvo] (NHD) or [Hkv, kv_len, D]
    (HND); v may be k or its prefix view k[..., :Dvo].  custom_mask [qo_len, kv_len] bool (False =
    masked) takes precedence over causal (bottom-right).  Returns out [qo_len, Hq, Dvo], or
    (out, lse [qo_len, Hq]) with return_lse."""
    binding.load()
    if q.dtype not in _TORCH_DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise binding.SfaError("sfa_prefill", 2)
    if kv_layout not in binding.KV_LAYOUT:
        raise binding.SfaError("sfa_prefill", 3)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be 3-d tensors")
    qo_len, Hq, Dqk = q.shape
    if kv_layout == "NHD":
        kv_len, Hkv = k.shape[0], k.shape[1]
        want_v = (kv_len, Hkv, v.shape[-1])
        ks, vs = (k.stride(0), k.stride(1)), (v.stride(0), v.stride(1))
    else:
        Hkv, kv_len = k.shape[0], k.shape[1]
        want_v = (Hkv, kv_len, v.shape[-1])
        ks, vs = (k.stride(1), k.stride(0)), (v.stride(1), v.stride(0))
    Dvo = v.shape[-1]
    if k.shape[-1] != Dqk or tuple(v.shape) != want_v:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)} in {kv_layout}")
    if custom_mask is not None and tuple(custom_mask.shape) != (qo_len, kv_len):
        raise ValueError(f"custom_mask must have shape {(qo_len, kv_len)}")
    if not q.is_contiguous() or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise binding.SfaError("sfa_prefill", 3)
    if not q.is_cuda:
        raise ValueError("single_prefill_with_kv_cache runs on the GPU: pass device tensors")
    dev = q.device
    for name, t in (("k", k), ("v", v)):
        _check_device_tensor(name, t, dev)
    mask_u8 = None
    if custom_mask is not None:
        _check_device_tensor("custom_mask", custom_mask, dev)
        # bool storage is one byte per element holding 0 or 1, which the library reads as uint8
        mask_u8 = custom_mask if custom_mask.dtype in (torch.bool, torch.uint8) and custom_mask.is_contiguous() \
            else (custom_mask != 0).contiguous()
    if out is None:
        out = torch.empty((qo_len, Hq, Dvo), dtype=q.dtype, device=dev)
    elif tuple(out.shape) != (qo_len, Hq, Dvo) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {q.dtype} tensor of shape {(qo_len, Hq, Dvo)}")
    _check_device_tensor("out", out, dev)
    if return_lse and lse is None:
        lse = torch.empty((qo_len, Hq), dtype=torch.float32, device=dev)
    _check_lse("sfa_prefill", lse, (qo_len, Hq), dev)
    need = binding.sfa_prefill_workspace_bytes(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, mask_u8 is not None)
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check_device_tensor("workspace", workspace, dev)
    rc = binding.sfa_prefill(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, binding.DTYPE[_TORCH_DTYPES[q.dtype]],
                             binding.KV_LAYOUT[kv_layout], ks + vs, int(bool(causal)), float(sm_scale or 0.0),
                             q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             mask_u8.data_ptr() if mask_u8 is not None else None, out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, workspace.data_ptr(), _nbytes(workspace),
                             _stream_handle())
    _check("sfa_prefill", rc)
    return (out, lse) if return_lse else out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
