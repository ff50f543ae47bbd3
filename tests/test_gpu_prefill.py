"""GPU parity of the dense prefill call (single_prefill_with_kv_cache page: custom_mask, causal,
kv_layout) against the fp64 oracle's dense masked attention."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import precision
from sparse_attention_13_amd import api

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _check(o, lse, q, k, v, mask, causal, dtype, rows=None, tag=""):
    """k / v in NHD for the oracle."""
    g_y, g_lse = oracle.dense_masked(q, k, v, mask=mask, causal=causal, rows=rows)
    Dvo = v.shape[-1]
    yb = o.reshape(-1, Dvo).float().cpu().numpy()
    lb = lse.reshape(-1).cpu().numpy()
    if rows is not None:
        yb, lb = yb[rows], lb[rows]
    rep = precision.gate(yb, g_y, dtype)
    log(f"  {tag} gate: {rep}")
    assert rep["pass"], rep
    fin = np.isfinite(g_lse)
    assert np.array_equal(np.isfinite(lb), fin)
    np.testing.assert_allclose(lb[fin], g_lse[fin], rtol=2e-6, atol=2e-6)
    if (~fin).any():
        assert np.all(yb[~fin] == 0.0)  # a row with no allowed key outputs +0
    return rep


def test_page_example_causal_and_tril_mask():
    # the page's example: qo_len 128, kv_len 4096, 32 query heads on 4 KV heads, head dim 128, fp16;
    # causal=True equals the custom mask tril(ones, diagonal = kv_len - qo_len)
    qo, kv, Hq, Hkv, D = 128, 4096, 32, 4, 128
    log(f"prefill page example qo={qo} kv={kv} Hq={Hq} Hkv={Hkv} D={D}")
    q, k, v = _rand((qo, Hq, D), 1, torch.float16), _rand((kv, Hkv, D), 2, torch.float16), \
        _rand((kv, Hkv, D), 3, torch.float16)
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = api.single_prefill_with_kv_cache(dq, dk, dv, causal=True, return_lse=True)
    mask = torch.tril(torch.full((qo, kv), True), diagonal=kv - qo)
    o2, lse2 = api.single_prefill_with_kv_cache(dq, dk, dv, custom_mask=mask.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    assert o.shape == (qo, Hq, D)
    # the same keys are masked either way, so every exponent and sum is the same
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    _check(o, lse, q, k, v, None, True, "fp16", tag="causal")
    _check(o2, lse2, q, k, v, mask, False, "fp16", tag="tril mask")


@pytest.mark.parametrize("density", [0.5, 0.05])
def test_page_shape_random_mask(density):
    qo, kv, Hq, Hkv, D = 128, 4096, 32, 4, 128
    log(f"prefill random mask density={density}")
    q, k, v = _rand((qo, Hq, D), 4, torch.float16), _rand((kv, Hkv, D), 5, torch.float16), \
        _rand((kv, Hkv, D), 6, torch.float16)
    g = torch.Generator().manual_seed(7)
    mask = torch.rand((qo, kv), generator=g) < density
    mask[5] = False  # a query row with no allowed key
    o, lse = api.single_prefill_with_kv_cache(q.to(DEV), k.to(DEV), v.to(DEV), custom_mask=mask.to(DEV),
                                              causal=True, return_lse=True)  # causal is ignored with a mask
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, mask, False, "fp16", tag=f"random mask {density}")


@pytest.mark.parametrize("qo,kv,Hq,Hkv,Dqk,Dvo,layout,dtype,causal,masked,value", [
    (77, 300, 8, 2, 128, 128, "NHD", "bf16", True, False, "separate"),    # ragged rows and keys
    (77, 300, 8, 2, 128, 128, "HND", "bf16", False, True, "separate"),
    (200, 333, 16, 1, 192, 128, "NHD", "fp16", True, False, "prefix"),    # value = key[..., :128]
    (64, 256, 4, 4, 64, 64, "HND", "fp16", False, True, "same"),          # value is key, MHA
    (33, 96, 32, 1, 512, 512, "NHD", "bf16", False, True, "same"),        # wide values, masked
    (40, 700, 64, 1, 576, 512, "NHD", "bf16", True, False, "prefix"),     # MLA-like, causal
    (16, 16, 2, 1, 320, 256, "HND", "fp16", True, True, "separate"),      # padded head dims
])
def test_shapes(qo, kv, Hq, Hkv, Dqk, Dvo, layout, dtype, causal, masked, value):
    dt = torch.float16 if dtype == "fp16" else torch.bfloat16
    log(f"prefill qo={qo} kv={kv} Hq={Hq} Hkv={Hkv} Dqk={Dqk} Dvo={Dvo} {layout} {dtype} causal={causal} "
        f"masked={masked} v={value}")
    q = _rand((qo, Hq, Dqk), 11, dt)
    k = _rand((kv, Hkv, Dqk), 12, dt)
    if value == "separate":
        v = _rand((kv, Hkv, Dvo), 13, dt)
    else:
        v = k[..., :Dvo]
    mask = None
    if masked:
        g = torch.Generator().manual_seed(14)
        mask = torch.rand((qo, kv), generator=g) < 0.4
    if layout == "NHD":
        dk = k.to(DEV)
        dv = dk[..., :Dvo] if value != "separate" else v.to(DEV)
    else:
        dk = k.permute(1, 0, 2).contiguous().to(DEV)
        dv = dk[..., :Dvo] if value != "separate" else v.permute(1, 0, 2).contiguous().to(DEV)
    o, lse = api.single_prefill_with_kv_cache(q.to(DEV), dk, dv, custom_mask=None if mask is None else mask.to(DEV),
                                              causal=causal, kv_layout=layout, return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v.contiguous(), mask, causal and mask is None, dtype)



@pytest.mark.parametrize("masked,value", [(False, "separate"), (True, "separate"), (False, "prefix")])
def test_many_items(masked, value):
    """Enough work items (128 row blocks x 2 KV heads) that every key list stays whole: causal items
    of 32 rows x 8 heads run 1 to 128 ring chunks on the eight-wave kernel (the deep pipeline),
    Dqk 192, Dvo 128, with separate values or V = K[..., :128]; sampled rows against the oracle."""
    qo, kv, Hq, Hkv, Dqk, Dvo = 4096, 4096, 16, 2, 192, 128
    log(f"prefill many items qo={qo} kv={kv} Hq={Hq} Hkv={Hkv} Dqk={Dqk} Dvo={Dvo} masked={masked} v={value}")
    q = _rand((qo, Hq, Dqk), 41, torch.bfloat16)
    k = _rand((kv, Hkv, Dqk), 42, torch.bfloat16)
    v = _rand((kv, Hkv, Dvo), 43, torch.bfloat16) if value == "separate" else k[..., :Dvo]
    mask = None
    if masked:
        g = torch.Generator().manual_seed(44)
        mask = torch.rand((qo, kv), generator=g) < 0.3
    dk = k.to(DEV)
    dv = v.to(DEV) if value == "separate" else dk[..., :Dvo]
    o, lse = api.single_prefill_with_kv_cache(q.to(DEV), dk, dv, custom_mask=None if mask is None else mask.to(DEV),
                                              causal=not masked, return_lse=True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(45).choice(qo * Hq, size=768, replace=False))
    _check(o, lse, q, k, v.contiguous(), mask, not masked, "bf16", rows=rows, tag="many items")

def test_rejects_bad_arguments():
    q = torch.zeros((8, 4, 64), dtype=torch.float16, device=DEV)
    k = torch.zeros((4, 2, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(Exception) as e:  # causal with more query rows than keys and no mask
        api.single_prefill_with_kv_cache(q, k, k, causal=True)
    assert "CAUSAL" in str(e.value)
    with pytest.raises(ValueError):
        api.single_prefill_with_kv_cache(q, k, k, custom_mask=torch.ones((8, 5), dtype=torch.bool, device=DEV))
    with pytest.raises(ValueError):
        api.single_prefill_with_kv_cache(q, k[..., :32].contiguous(), k)
