"""The allocation-free variant of sfa_run (split-K partials in the library's own device array)
against sfa_run with a caller workspace, through the C ABI: two calls in a row, the second with a
smaller problem, both bitwise equal to sfa_run's results (same kernels, same plan)."""
import ctypes
import sys

import pytest
import torch

from sparse_attention_13_amd import api, binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp, Dv):
    k = inp["k"].to(DEV)
    v = k if inp["v"] is inp["k"] else (k[..., :Dv] if inp["v"].data_ptr() == inp["k"].data_ptr()
                                        else inp["v"].to(DEV))
    return inp["q"].to(DEV), k, v, inp["idx"].to(DEV)


def _noalloc(shape, q, k, v, idx, out, lse):
    sh = api.sfa_shape_of(q, k, v, idx, shape.layout)
    st = binding.make_strides(q.stride(), k.stride(), v.stride(), idx.stride(), out.stride())
    return binding.sfa_run_noalloc(sh, st, binding.DTYPE[shape.dtype], binding.LAYOUT[shape.layout],
                                   int(shape.causal), shape.scale_value, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   idx.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)


def _case(shape, seed):
    print(f"no-alloc case {shape}", flush=True)
    inp = synth.sfa_inputs(shape, seed)
    q, k, v, idx = _dev(inp, shape.Dv)
    ref, ref_lse = api.sparse_flash_attention(q, k, v, idx, shape.scale_value, shape.layout, shape.causal,
                                              return_lse=True)
    out, lse = torch.full_like(ref, float("nan")), torch.full_like(ref_lse, float("nan"))
    assert _noalloc(shape, q, k, v, idx, out, lse) == binding.SFA_OK
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_matches_sfa_run_twice_then_smaller():
    assert binding.sfa_run_noalloc_max_workspace() == 64 << 20
    # the MLA decode workload (split-K partials in the scratch array), then a smaller split problem
    _case(synth.WORKLOADS["mla_decode"], 3)
    _case(synth.SfaShape(B=2, S1=1, S2=4096, N1=16, N2=2, Dk=128, Dv=128, topK=1500, dtype="fp16",
                         layout="BNSD", causal=False), 4)


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 128 index lists of 16384 slots, each shared by 128 query heads with wide values: the lists
    # exceed what one work item stages, so every one is split and the partials need far more than
    # 64 MiB (checked on the host; nothing is launched)
    shape = binding.make_shape(8, 2, 16384, 1024, 8, 576, 512, 16384)
    need = binding.sfa_workspace_bytes(shape, 1, 0)
    assert need > 64 << 20
    rc = binding.sfa_run_noalloc(shape, None, 1, 1, 0, 0.04, 16, 16, 16, 16, 16, None, None)
    assert rc == 10
