"""ctypes binding of libsfa.so: the C ABI of include/sfa.h, one Python function per
exported symbol, with the same names and arguments (pointers as ints).

This module only marshals arguments.  It raises if the HIP library has not been
built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SFA_LIB", os.path.join(_PKG, "libsfa.so"))

SFA_OK = 0
STATUS = {
    0: "SFA_OK", 1: "SFA_ERR_NULL", 2: "SFA_ERR_DTYPE", 3: "SFA_ERR_LAYOUT", 4: "SFA_ERR_SHAPE",
    5: "SFA_ERR_GQA", 6: "SFA_ERR_HEAD_DIM", 7: "SFA_ERR_TOPK", 8: "SFA_ERR_CAUSAL", 9: "SFA_ERR_SCALE",
    10: "SFA_ERR_WORKSPACE", 11: "SFA_ERR_PLAN", 12: "SFA_ERR_INDEX", 13: "SFA_ERR_UNSUPPORTED",
    14: "SFA_ERR_HIP",
}
DTYPE = {"fp16": 0, "bf16": 1}
LAYOUT = {"BSND": 0, "BNSD": 1}
KV_LAYOUT = {"NHD": 0, "HND": 1}
FP8 = {"e4m3": 0, "e5m2": 1}

EXPORTS = ("sfa_workspace_bytes", "sfa_run", "bsr_plan_workspace_bytes", "bsr_plan_float_workspace_bytes",
           "bsr_plan", "bsr_run", "bsr_destroy", "vbsr_plan_workspace_bytes", "vbsr_plan_float_workspace_bytes",
           "vbsr_plan", "vbsr_run", "vbsr_destroy", "sfa_status_str",
           "bsr_fp8_workspace_bytes", "bsr_run_fp8", "vbsr_fp8_workspace_bytes", "vbsr_run_fp8",
           "sfa_validate_indices", "sfa_prefill_workspace_bytes", "sfa_prefill", "sfa_run_noalloc_max_workspace",
           "sfa_run_noalloc")


class SfaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "S1", "S2", "N1", "N2", "Dk", "Dv", "topK")]


class SfaStrides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64 * 3) for n in ("q", "k", "v", "idx", "out")]


class SfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status_str(status)})")


_lib = None
_lock = threading.Lock()


def load():
    """Loads libsfa.so once; raises RuntimeError when it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libsfa.so not found at {LIB_PATH}: build it with `python -m sparse_attention_13_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.sfa_workspace_bytes.argtypes = [ctypes.POINTER(SfaShape), I, I]
        lib.sfa_workspace_bytes.restype = Z
        lib.sfa_run.argtypes = [ctypes.POINTER(SfaShape), ctypes.POINTER(SfaStrides), I, I, I, F, P, P, P, P, P, P,
                                P, Z, P]
        lib.sfa_run.restype = I
        lib.bsr_plan_workspace_bytes.argtypes = [P, P, P, I, I, I, I, I, I, I]
        lib.bsr_plan_workspace_bytes.restype = Z
        lib.bsr_plan_float_workspace_bytes.argtypes = [P, P, I, I, I, I, I, I, I]
        lib.bsr_plan_float_workspace_bytes.restype = Z
        lib.bsr_plan.argtypes = [ctypes.POINTER(P), P, P, P, I, I, I, I, I, I, I, I, F, I, P, Z, P, Z, P]
        lib.bsr_plan.restype = I
        lib.bsr_run.argtypes = [P, P, P, P, P, P, P]
        lib.bsr_run.restype = I
        lib.bsr_destroy.argtypes = [P]
        lib.bsr_destroy.restype = I
        lib.vbsr_plan_workspace_bytes.argtypes = [P, P, P, I, I, I, I, I]
        lib.vbsr_plan_workspace_bytes.restype = Z
        lib.vbsr_plan_float_workspace_bytes.argtypes = [P, P, P, I, I, I, I, I]
        lib.vbsr_plan_float_workspace_bytes.restype = Z
        lib.vbsr_plan.argtypes = [ctypes.POINTER(P), P, P, P, I, I, I, I, I, I, F, I, P, Z, P, Z, P]
        lib.vbsr_plan.restype = I
        lib.vbsr_run.argtypes = [P, P, P, P, P, P, P]
        lib.vbsr_run.restype = I
        lib.vbsr_destroy.argtypes = [P]
        lib.vbsr_destroy.restype = I
        for pre in ("bsr", "vbsr"):
            getattr(lib, pre + "_fp8_workspace_bytes").argtypes = [P]
            getattr(lib, pre + "_fp8_workspace_bytes").restype = Z
            getattr(lib, pre + "_run_fp8").argtypes = [P, P, P, P, I, I, P, P, P, P, P, P, Z, P]
            getattr(lib, pre + "_run_fp8").restype = I
        lib.sfa_validate_indices.argtypes = [ctypes.POINTER(SfaShape), ctypes.POINTER(SfaStrides), I, P, P, P]
        lib.sfa_validate_indices.restype = I
        lib.sfa_prefill_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.sfa_prefill_workspace_bytes.restype = Z
        lib.sfa_prefill.argtypes = [I, I, I, I, I, I, I, I, P, I, F, P, P, P, P, P, P, P, Z, P]
        lib.sfa_prefill.restype = I
        lib.sfa_run_noalloc_max_workspace.argtypes = []
        lib.sfa_run_noalloc_max_workspace.restype = Z
        lib.sfa_run_noalloc.argtypes = [ctypes.POINTER(SfaShape), ctypes.POINTER(SfaStrides), I, I, I, F, P, P, P, P,
                                        P, P, P]
        lib.sfa_run_noalloc.restype = I
        lib.sfa_status_str.argtypes = [I]
        lib.sfa_status_str.restype = ctypes.c_char_p
        _lib = lib
        return lib


def status_str(status: int) -> str:
    try:
        return load().sfa_status_str(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def make_shape(B, S1, S2, N1, N2, Dk, Dv, topK) -> SfaShape:
    return SfaShape(B, S1, S2, N1, N2, Dk, Dv, topK)


def make_strides(q, k, v, idx, out) -> SfaStrides:
    s = SfaStrides()
    for name, st in (("q", q), ("k", k), ("v", v), ("idx", idx), ("out", out)):
        arr = getattr(s, name)
        for i in range(3):
            arr[i] = int(st[i])
    return s


def sfa_workspace_bytes(shape: SfaShape, dtype: int, causal: int) -> int:
    return int(load().sfa_workspace_bytes(ctypes.byref(shape), int(dtype), int(causal)))


def sfa_run(shape: SfaShape, strides, dtype: int, layout: int, causal: int, scale: float, q: int, k: int, v: int,
            sparse_indices: int, out: int, lse, workspace, workspace_bytes: int, stream) -> int:
    st = ctypes.byref(strides) if strides is not None else None
    return int(load().sfa_run(ctypes.byref(shape), st, int(dtype), int(layout), int(causal), float(scale),
                              q, k, v, sparse_indices, out, lse, workspace, int(workspace_bytes), stream))


def sfa_run_prepared(shape: SfaShape, strides, dtype: int, layout: int, causal: int, scale: float, q: int, k: int,
                     v: int, sparse_indices: int, out: int, lse, workspace, workspace_bytes: int):
    """Returns (foreign function, converted argument tuple without the stream) for repeated launches."""
    lib = load()
    st = ctypes.byref(strides) if strides is not None else None
    args = (ctypes.byref(shape), st, ctypes.c_int(dtype), ctypes.c_int(layout), ctypes.c_int(causal),
            ctypes.c_float(scale), ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v),
            ctypes.c_void_p(sparse_indices), ctypes.c_void_p(out), ctypes.c_void_p(lse),
            ctypes.c_void_p(workspace), ctypes.c_size_t(workspace_bytes))
    return lib.sfa_run, args


def sfa_validate_indices(shape: SfaShape, strides, layout: int, sparse_indices: int, counts: int, stream) -> int:
    st = ctypes.byref(strides) if strides is not None else None
    sh = ctypes.byref(shape) if shape is not None else None
    return int(load().sfa_validate_indices(sh, st, int(layout), sparse_indices, counts, stream))


def bsr_plan_workspace_bytes(indptr: int, indices: int, M, N, R, C, Hq, Hkv, D, mask: Optional[int] = None) -> int:
    return int(load().bsr_plan_workspace_bytes(indptr, indices, mask, M, N, R, C, Hq, Hkv, D))


def bsr_plan_float_workspace_bytes(indptr: int, indices: int, M, N, R, C, Hq, Hkv, D) -> int:
    return int(load().bsr_plan_float_workspace_bytes(indptr, indices, M, N, R, C, Hq, Hkv, D))


def bsr_plan(indptr: int, indices: int, M, N, R, C, Hq, Hkv, D, causal, sm_scale, dtype, workspace: int,
             workspace_bytes: int, stream, mask: Optional[int] = None, float_workspace: Optional[int] = None,
             float_workspace_bytes: int = 0):
    """Returns (status, plan_handle).  mask: host address of a [nnz, R, C] uint8 block mask, or None."""
    handle = ctypes.c_void_p()
    rc = int(load().bsr_plan(ctypes.byref(handle), indptr, indices, mask, M, N, R, C, Hq, Hkv, D, int(causal),
                             float(sm_scale), int(dtype), workspace, int(workspace_bytes), float_workspace,
                             int(float_workspace_bytes), stream))
    return rc, handle.value


def bsr_run(plan: int, q: int, k: int, v: int, out: int, lse, stream) -> int:
    return int(load().bsr_run(plan, q, k, v, out, lse, stream))


def bsr_destroy(plan) -> int:
    return int(load().bsr_destroy(plan))


def vbsr_plan_workspace_bytes(block_mask_map: int, block_row_sz: int, block_col_sz: int, Hkv, MB, NB, Hq, D) -> int:
    return int(load().vbsr_plan_workspace_bytes(block_mask_map, block_row_sz, block_col_sz, Hkv, MB, NB, Hq, D))


def vbsr_plan_float_workspace_bytes(block_mask_map: int, block_row_sz: int, block_col_sz: int, Hkv, MB, NB, Hq,
                                    D) -> int:
    return int(load().vbsr_plan_float_workspace_bytes(block_mask_map, block_row_sz, block_col_sz, Hkv, MB, NB, Hq, D))


def vbsr_plan(block_mask_map: int, block_row_sz: int, block_col_sz: int, Hkv, MB, NB, Hq, D, causal, sm_scale,
              dtype, workspace: int, workspace_bytes: int, stream, float_workspace: Optional[int] = None,
              float_workspace_bytes: int = 0):
    """Returns (status, plan_handle); the pattern arguments are host addresses."""
    handle = ctypes.c_void_p()
    rc = int(load().vbsr_plan(ctypes.byref(handle), block_mask_map, block_row_sz, block_col_sz, Hkv, MB, NB, Hq, D,
                              int(causal), float(sm_scale), int(dtype), workspace, int(workspace_bytes),
                              float_workspace, int(float_workspace_bytes), stream))
    return rc, handle.value


def vbsr_run(plan: int, q: int, k: int, v: int, out: int, lse, stream) -> int:
    return int(load().vbsr_run(plan, q, k, v, out, lse, stream))


def vbsr_destroy(plan) -> int:
    return int(load().vbsr_destroy(plan))


def bsr_fp8_workspace_bytes(plan) -> int:
    return int(load().bsr_fp8_workspace_bytes(plan))


def bsr_run_fp8(plan, q: int, k: int, v: int, q_fmt: int, kv_fmt: int, scale_q, scale_k, scale_v, out: int, lse,
                workspace, workspace_bytes: int, stream) -> int:
    return int(load().bsr_run_fp8(plan, q, k, v, int(q_fmt), int(kv_fmt), scale_q, scale_k, scale_v, out, lse,
                                  workspace, int(workspace_bytes), stream))


def vbsr_fp8_workspace_bytes(plan) -> int:
    return int(load().vbsr_fp8_workspace_bytes(plan))


def vbsr_run_fp8(plan, q: int, k: int, v: int, q_fmt: int, kv_fmt: int, scale_q, scale_k, scale_v, out: int, lse,
                 workspace, workspace_bytes: int, stream) -> int:
    return int(load().vbsr_run_fp8(plan, q, k, v, int(q_fmt), int(kv_fmt), scale_q, scale_k, scale_v, out, lse,
                                   workspace, int(workspace_bytes), stream))


def sfa_prefill_workspace_bytes(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, masked) -> int:
    return int(load().sfa_prefill_workspace_bytes(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, int(bool(masked))))


def sfa_prefill(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, dtype: int, kv_layout: int, kv_strides, causal, sm_scale,
                q: int, k: int, v: int, mask, out: int, lse, workspace, workspace_bytes: int, stream) -> int:
    """kv_strides: None or four ints (k row, k head, v row, v head)."""
    st = (ctypes.c_int64 * 4)(*[int(x) for x in kv_strides]) if kv_strides is not None else None
    return int(load().sfa_prefill(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, int(dtype), int(kv_layout), st, int(causal),
                                  float(sm_scale), q, k, v, mask, out, lse, workspace, int(workspace_bytes), stream))


def sfa_run_noalloc_max_workspace() -> int:
    return int(load().sfa_run_noalloc_max_workspace())


def sfa_run_noalloc(shape: SfaShape, strides, dtype: int, layout: int, causal: int, scale: float, q: int, k: int,
                    v: int, sparse_indices: int, out: int, lse, stream) -> int:
    st = ctypes.byref(strides) if strides is not None else None
    return int(load().sfa_run_noalloc(ctypes.byref(shape), st, int(dtype), int(layout), int(causal), float(scale),
                                      q, k, v, sparse_indices, out, lse, stream))
