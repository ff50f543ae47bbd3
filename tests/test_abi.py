"""CPU checks of the C ABI: the library loads, exports every declared symbol, and
rejects each rule violation with its status code before touching a device."""
import ctypes
import os
import re

import pytest

from sparse_attention_13_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from sparse_attention_13_amd import build
        build.build(verbose=False)
    return binding.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sfa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(\w+)\s*\(", text)) & set(
        n for n in re.findall(r"\b(sfa_\w+|v?bsr_\w+)\b", text))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert {"sfa_run", "sfa_workspace_bytes", "bsr_plan", "bsr_run", "bsr_destroy", "sfa_status_str",
            "bsr_plan_workspace_bytes", "vbsr_plan_workspace_bytes", "vbsr_plan", "vbsr_run",
            "vbsr_destroy"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(binding.EXPORTS) == declared


def test_status_strings(lib):
    for code in binding.STATUS:
        assert len(binding.status_str(code)) > 0


BASE = dict(B=1, S1=4, S2=64, N1=4, N2=1, Dk=64, Dv=64, topK=16)
FAKE = 1 << 20  # 16-byte aligned non-null stand-in pointer; never dereferenced on these paths


def _run(lib, dtype=0, layout=0, causal=0, scale=0.125, ptrs=None, **kw):
    sh = dict(BASE)
    sh.update(kw)
    shape = binding.make_shape(**sh)
    p = ptrs or [FAKE] * 5
    return binding.sfa_run(shape, None, dtype, layout, causal, scale, *p, None, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 2),
    (dict(layout=5), 3),
    (dict(S2=0), 4),
    (dict(B=-1), 4),
    (dict(N2=0), 4),
    (dict(N1=6, N2=4), 5),
    (dict(Dk=96), 6),
    (dict(Dv=128), 6),  # Dv > Dk
    (dict(Dk=0), 6),
    (dict(topK=0), 7),
    (dict(topK=65), 7),
    (dict(causal=1, S1=65, topK=16), 8),
    (dict(scale=0.0), 9),
    (dict(scale=-1.0), 9),
    (dict(scale=float("inf")), 9),
    (dict(scale=float("nan")), 9),
    (dict(ptrs=[0, FAKE, FAKE, FAKE, FAKE]), 1),
    (dict(ptrs=[FAKE, FAKE, FAKE, FAKE, 0]), 1),
    (dict(ptrs=[FAKE + 2, FAKE, FAKE, FAKE, FAKE]), 3),  # misaligned rows
    (dict(Dk=640, Dv=64), 13),  # head dim above the widest the page lists (576)
])
def test_rule_violations_are_rejected(lib, kw, code):
    assert _run(lib, **kw) == code


def test_empty_batch_is_a_noop(lib):
    assert _run(lib, B=0) == 0
    assert _run(lib, S1=0) == 0


def test_null_shape(lib):
    assert lib.sfa_run(None, None, 0, 0, 0, 1.0, None, None, None, None, None, None, None, 0, None) == 1


def _plan(lib, indptr, indices, M=4, N=4, R=2, C=2, Hq=4, Hkv=2, D=64, causal=0, ws=FAKE, ws_bytes=1 << 20,
          fws=None, fws_bytes=0):
    import torch
    ip = torch.tensor(indptr, dtype=torch.int32)
    ix = torch.tensor(indices if indices else [0], dtype=torch.int32)
    rc, handle = binding.bsr_plan(ip.data_ptr(), ix.data_ptr(), M, N, R, C, Hq, Hkv, D, causal, 0.0, 0, ws, ws_bytes,
                                  None, None, fws, fws_bytes)
    assert handle is None
    return rc


@pytest.mark.parametrize("kw,code", [
    (dict(indptr=[0, 2, 3], indices=[0, 0, 1]), 12),        # repeated column block in a block row
    (dict(indptr=[0, 1, 2], indices=[0, 2]), 12),           # column block >= N / C
    (dict(indptr=[0, 1, 2], indices=[0, -1]), 12),
    (dict(indptr=[1, 1, 2], indices=[0, 1]), 11),           # indptr[0] != 0
    (dict(indptr=[0, 2, 1], indices=[0, 1]), 11),           # decreasing indptr
    (dict(indptr=[0, 1, 2], indices=[0, 1], N=5), 4),       # N % C != 0
    (dict(indptr=[0, 1, 2], indices=[0, 1], Hq=3), 5),      # Hq % Hkv != 0
    (dict(indptr=[0, 1, 2], indices=[0, 1], D=96), 6),
    (dict(indptr=[0, 1, 2], indices=[0, 1], D=640), 13),    # head dim above 576
    (dict(indptr=[0, 1, 2], indices=[0, 1], M=5, causal=1), 8),
    (dict(indptr=[0, 1, 2], indices=[0, 1], ws=0), 10),
    (dict(indptr=[0, 1, 2], indices=[0, 1], ws_bytes=8), 10),
])
def test_bsr_plan_rejects(lib, kw, code):
    assert _plan(lib, **kw) == code


def test_bsr_run_without_plan(lib):
    assert binding.bsr_run(None, FAKE, FAKE, FAKE, FAKE, None, None) == 11
    assert binding.bsr_destroy(None) == 0


def _vplan(bmap, rs, cs, Hq=4, D=64, causal=0, ws=FAKE, ws_bytes=1 << 20, fws=None, fws_bytes=0):
    import torch
    bm = torch.tensor(bmap, dtype=torch.uint8)
    r = torch.tensor(rs, dtype=torch.int32)
    c = torch.tensor(cs, dtype=torch.int32)
    Hkv, MB, NB = bm.shape
    rc, handle = binding.vbsr_plan(bm.data_ptr(), r.data_ptr(), c.data_ptr(), Hkv, MB, NB, Hq, D, causal, 0.0, 0,
                                   ws, ws_bytes, None, fws, fws_bytes)
    assert handle is None
    return rc


_VB = dict(bmap=[[[1, 0], [0, 1]], [[1, 1], [0, 1]]], rs=[[2, 3], [4, 1]], cs=[[3, 3], [1, 5]])


@pytest.mark.parametrize("kw,code", [
    (dict(rs=[[2, 3], [4, 2]]), 4),                  # heads cover different query lengths
    (dict(cs=[[3, 3], [2, 5]]), 4),                  # heads cover different key lengths
    (dict(rs=[[2, 3], [6, -1]]), 4),                 # negative size
    (dict(cs=[[0, 0], [0, 0]]), 4),                  # no keys (N = 0)
    (dict(Hq=3), 5),                                 # Hq % Hkv != 0
    (dict(D=96), 6),
    (dict(D=640), 13),                               # head dim above 576
    (dict(rs=[[5, 3], [4, 4]], cs=[[3, 4], [1, 6]], causal=1), 8),   # causal with M > N
    (dict(ws=0), 10),
    (dict(ws_bytes=8), 10),
])
def test_vbsr_plan_rejects(lib, kw, code):
    args = {**_VB, **kw}
    assert _vplan(**args) == code


def test_vbsr_workspace_bytes_and_null_plan(lib):
    import torch
    bm = torch.tensor(_VB["bmap"], dtype=torch.uint8)
    r = torch.tensor(_VB["rs"], dtype=torch.int32)
    c = torch.tensor(_VB["cs"], dtype=torch.int32)
    assert binding.vbsr_plan_workspace_bytes(bm.data_ptr(), r.data_ptr(), c.data_ptr(), 2, 2, 2, 4, 64) > 0
    assert binding.vbsr_plan_workspace_bytes(bm.data_ptr(), r.data_ptr(), c.data_ptr(), 2, 2, 2, 3, 64) == 0
    assert binding.vbsr_plan_workspace_bytes(None, None, c.data_ptr(), 2, 2, 2, 4, 64) == 0
    assert binding.vbsr_run(None, FAKE, FAKE, FAKE, FAKE, None, None) == 11
    assert binding.vbsr_destroy(None) == 0


def test_fp8_runs_without_plan(lib):
    assert binding.bsr_fp8_workspace_bytes(None) == 0
    assert binding.vbsr_fp8_workspace_bytes(None) == 0
    for fn in (binding.bsr_run_fp8, binding.vbsr_run_fp8):
        assert fn(None, FAKE, FAKE, FAKE, 0, 0, None, None, None, FAKE, None, FAKE, 1 << 20, None) == 11


def test_validate_indices_rejects(lib):
    shape = binding.make_shape(1, 2, 10, 2, 2, 64, 64, 4)
    assert binding.sfa_validate_indices(None, None, 0, FAKE, FAKE, None) == 1
    assert binding.sfa_validate_indices(shape, None, 7, FAKE, FAKE, None) == 3
    assert binding.sfa_validate_indices(shape, None, 0, FAKE, None, None) == 1
    assert binding.sfa_validate_indices(binding.make_shape(1, 2, 10, 2, 2, 64, 64, 11), None, 0, FAKE, FAKE,
                                        None) == 7
    assert binding.sfa_validate_indices(binding.make_shape(1, 2, 1 << 21, 2, 2, 64, 64, 4), None, 0, FAKE, FAKE,
                                        None) == 13


def _long_rows_pattern():
    """One block row of 64 column blocks and one KV head: a single long key list, which the plan
    splits (so its runs need the float workspace for the split partials)."""
    import torch
    ip = torch.tensor([0, 64], dtype=torch.int32)
    ix = torch.arange(64, dtype=torch.int32)
    return ip, ix, dict(M=2, N=4096, R=2, C=64, Hq=4, Hkv=1, D=64)


def test_bsr_float_workspace_is_the_split_scratch(lib):
    ip, ix, g = _long_rows_pattern()
    args = (ip.data_ptr(), ix.data_ptr(), g["M"], g["N"], g["R"], g["C"], g["Hq"], g["Hkv"], g["D"])
    need_f = binding.bsr_plan_float_workspace_bytes(*args)
    need_i = binding.bsr_plan_workspace_bytes(*args)
    assert need_f > 0 and need_i > 0
    # key lists only in the int workspace
    assert need_i < 64 * 64 * 4 + 4096
    plan = lambda fws, fb: _plan(lib, [0, 64], list(range(64)), fws=fws, fws_bytes=fb, **g)
    assert plan(None, 0) == 10
    assert plan(FAKE, need_f - 1) == 10
    # a pattern whose lists are not split needs no float workspace
    assert binding.bsr_plan_float_workspace_bytes(ip.data_ptr(), ix.data_ptr(), 64, 64, 64, 64, 4, 1, 64) == 0


def test_vbsr_float_workspace_is_the_split_scratch(lib):
    import torch
    bm = torch.ones((1, 1, 64), dtype=torch.uint8)
    r = torch.tensor([[2]], dtype=torch.int32)
    c = torch.full((1, 64), 64, dtype=torch.int32)
    need_f = binding.vbsr_plan_float_workspace_bytes(bm.data_ptr(), r.data_ptr(), c.data_ptr(), 1, 1, 64, 4, 64)
    assert need_f > 0
    assert _vplan(bm.tolist(), r.tolist(), c.tolist(), fws=None) == 10
    assert _vplan(bm.tolist(), r.tolist(), c.tolist(), fws=FAKE, fws_bytes=need_f - 1) == 10
