"""GPU parity of the top-K sparse attention kernels against the fp64 oracle.

Every comparison is element by element on the same seeded inputs, judged by the
SparseFlashAttention page's precision standard (oracle.precision.gate); mask and
index decisions are checked bit-exactly where the exact answer is known.
"""
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import precision
from sparse_attention_13_amd import api, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    k = inp["k"].to(DEV)
    if inp["v"] is inp["k"]:
        v = k
    elif inp["v"].data_ptr() == inp["k"].data_ptr():
        v = k[..., : inp["v"].shape[-1]]
    else:
        v = inp["v"].to(DEV)
    return inp["q"].to(DEV), k, v, inp["idx"].to(DEV)


def gpu_rows_bsnd(y, layout):
    """[B,S1,N1,Dv] view in (b, s1, n1) row order."""
    return y if layout == "BSND" else y.permute(0, 2, 1, 3)


def run_and_compare(shape: synth.SfaShape, seed=0, rows=None, check_lse=True, inp=None):
    log(f"case {shape} seed={seed} rows={'all' if rows is None else len(rows)}")
    if inp is None:
        inp = synth.sfa_inputs(shape, seed)
    q, k, v, idx = to_dev(inp)
    y, lse = api.sparse_flash_attention(q, k, v, idx, shape.scale_value, shape.layout, shape.causal,
                                        return_lse=True)
    torch.cuda.synchronize()
    yb = gpu_rows_bsnd(y, shape.layout).reshape(-1, shape.Dv).float().cpu().numpy()
    lb = (lse if shape.layout == "BSND" else lse.permute(0, 2, 1)).reshape(-1).cpu().numpy()
    g_y, g_lse = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], shape.scale_value, shape.layout,
                            shape.causal, rows=rows)
    if rows is not None:
        yb, lb = yb[rows], lb[rows]
    rep = precision.gate(yb, g_y, shape.dtype)
    log(f"  gate: {rep}")
    if os.environ.get("SFA_PARITY_LOG"):
        with open(os.environ["SFA_PARITY_LOG"], "a") as f:
            f.write(json.dumps({"case": str(shape), "seed": seed, "rows": "all" if rows is None else len(rows),
                                **{k: v for k, v in rep.items()}}) + "\n")
    assert rep["pass"], rep
    fin = np.isfinite(g_lse)
    assert np.array_equal(np.isfinite(lb), fin)
    if check_lse:
        np.testing.assert_allclose(lb[fin], g_lse[fin], rtol=2e-6, atol=2e-6)
    # fully masked rows: +0.0 exactly
    dead = ~fin
    if dead.any():
        assert np.all(yb[dead] == 0.0) and not np.any(np.signbit(yb[dead]))
    return rep


SMALL = [
    # (B, S1, S2, N1, N2, Dk, Dv, topK, dtype, layout, causal, value)
    (1, 4, 64, 4, 1, 64, 64, 16, "fp16", "BSND", False, "alias"),          # tiny workload geometry
    (2, 3, 300, 8, 2, 128, 128, 77, "bf16", "BSND", False, "alias"),       # ragged topK
    (2, 5, 257, 16, 2, 128, 128, 200, "fp16", "BNSD", True, "alias"),      # G=8, causal
    (1, 2, 500, 32, 1, 192, 128, 130, "fp16", "BSND", True, "alias"),      # G=32 -> 2 head tiles
    (1, 2, 400, 24, 1, 192, 128, 96, "bf16", "BNSD", False, "separate"),   # G=24 padded, separate V
    (2, 2, 600, 128, 1, 576, 512, 300, "bf16", "BNSD", True, "alias"),     # MLA geometry
    (1, 3, 200, 3, 3, 256, 256, 150, "fp16", "BSND", False, "separate"),   # G=1
    (1, 1, 1100, 2, 1, 512, 512, 1024, "bf16", "BSND", False, "alias"),    # G=2, large dims
    (3, 4, 90, 4, 2, 192, 192, 90, "fp16", "BSND", True, "separate"),      # topK == S2
    (1, 2, 5000, 8, 1, 128, 128, 2048, "bf16", "BSND", False, "alias"),    # longest topK
    (1, 1, 300, 64, 1, 576, 512, 100, "bf16", "BNSD", False, "separate"),  # wide dims, separate V: 16-wide tiles
    (2, 1, 700, 48, 2, 512, 512, 333, "fp16", "BSND", True, "alias"),      # G=24: one 32-wide tile, padded
    # many query vectors with wide values: PV split over dv (64 vectors per workgroup)
    (1, 2, 700, 96, 1, 576, 512, 200, "fp16", "BSND", True, "alias"),      # G=96: second block half empty
    (2, 1, 400, 64, 1, 512, 512, 150, "bf16", "BSND", False, "separate"),  # separate V, two-buffer ring
    (1, 1, 600, 128, 2, 512, 512, 257, "fp16", "BNSD", True, "alias"),     # two KV heads, ragged chunk
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_small_shapes_full_parity(case):
    B, S1, S2, N1, N2, Dk, Dv, topK, dt, layout, causal, value = case
    s = synth.SfaShape(B=B, S1=S1, S2=S2, N1=N1, N2=N2, Dk=Dk, Dv=Dv, topK=topK, dtype=dt, layout=layout,
                       causal=causal, value=value)
    run_and_compare(s, seed=1)


@pytest.mark.parametrize("name", ["tiny", "gqa_decode", "mla_decode", "gqa_prefill"])
def test_workloads_at_full_size(name):
    s = synth.WORKLOADS[name]
    nrows = s.B * s.S1 * s.N1
    if nrows <= 4096:
        rows = None
    else:
        g = np.random.default_rng(7)
        rows = np.sort(g.choice(nrows, size=2048, replace=False))
    run_and_compare(s, seed=0, rows=rows)


@pytest.mark.parametrize("case", [
    (2, 64, 256, 8, 2, 128, 128, "fp16", "BSND", "separate"),
    (1, 100, 333, 64, 1, 576, 512, "bf16", "BNSD", "alias"),
], ids=["gqa", "mla"])
def test_identity_indices_dense_causal(case):
    """topK = S2 with every key selected in order: dense attention with the bottom-right causal
    mask through the sparse kernels (the baseline the pages compare against), many tiles deep."""
    B, S1, S2, N1, N2, Dk, Dv, dt, layout, value = case
    s = synth.SfaShape(B=B, S1=S1, S2=S2, N1=N1, N2=N2, Dk=Dk, Dv=Dv, topK=S2, dtype=dt, layout=layout,
                       causal=True, value=value, sorted_indices=True)
    import dataclasses
    inp = synth.sfa_inputs(dataclasses.replace(s, topK=1), seed=4)
    ar = torch.arange(S2, dtype=torch.int32)
    shp = (B, S1, N2, S2) if layout == "BSND" else (B, N2, S1, S2)
    inp["idx"] = ar.view(1, 1, 1, S2).expand(*shp).contiguous()
    run_and_compare(s, seed=4, inp=inp)


def _custom(B, S1, S2, N1, N2, D, idx_rows, dtype=torch.float16, layout="BSND", causal=True, seed=3):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, S1, N1, D), generator=g).to(dtype)
    k = torch.randn((B, S2, N2, D), generator=g).to(dtype)
    v = torch.randn((B, S2, N2, D), generator=g).to(dtype)
    idx = None if idx_rows is None else torch.tensor(idx_rows, dtype=torch.int32)
    return q, k, v, idx


@pytest.mark.parametrize("N1,D", [(8, 128), (64, 512)])
def test_single_survivor_rows_are_exact(N1, D):
    """A row whose only unmasked slot is j outputs v[j] bit for bit; the masked decision is exact."""
    B, S1, S2, N2 = 1, 4, 40, 1
    survivors = {0: 5, 1: 12, 2: 7, 3: 20}
    rows = []
    for s1 in range(S1):
        limit = s1 + S2 - S1
        masked = list(range(limit + 1, S2))
        if masked:
            r = [masked[i % len(masked)] for i in range(32)]
            r[3 + s1] = survivors[s1]
        else:
            r = [survivors[s1]] * 32  # nothing maskable: 32 copies of one row
        rows.append(r)
    idx = torch.tensor(rows, dtype=torch.int32).view(B, S1, N2, 32)
    q, k, v, _ = _custom(B, S1, S2, N1, N2, D, None)
    y, lse = api.sparse_flash_attention(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), 0.3, "BSND", True,
                                        return_lse=True)
    y = y.cpu()
    for s1, j in survivors.items():
        for n1 in range(N1):
            assert torch.equal(y[0, s1, n1], v[0, j, 0]), (s1, n1)


@pytest.mark.parametrize("N1,N2,D", [(4, 2, 64), (128, 2, 512)])
def test_all_masked_rows_and_topk_one(N1, N2, D):
    B, S1, S2 = 2, 3, 10
    idx = torch.full((B, S1, N2, 1), 9, dtype=torch.int32)  # row s1 keeps idx <= s1 + 7: rows 0, 1 all masked
    q, k, v, _ = _custom(B, S1, S2, N1, N2, D, None)
    y, lse = api.sparse_flash_attention(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), 0.125, "BSND", True,
                                        return_lse=True)
    y, lse = y.cpu(), lse.cpu()
    assert torch.all(y[:, :2] == 0) and not torch.any(torch.signbit(y[:, :2].float()))
    assert torch.all(torch.isneginf(lse[:, :2]))
    G = N1 // N2
    for b in range(B):
        for n1 in range(N1):
            assert torch.equal(y[b, 2, n1], v[b, 9, n1 // G])
    # non-causal topK = 1: y == v[idx]
    idx1 = torch.randint(0, S2, (B, S1, N2, 1), dtype=torch.int32)
    y1 = api.sparse_flash_attention(q.to(DEV), k.to(DEV), v.to(DEV), idx1.to(DEV), 0.125, "BSND", False).cpu()
    for b in range(B):
        for s1 in range(S1):
            for n1 in range(N1):
                assert torch.equal(y1[b, s1, n1], v[b, int(idx1[b, s1, n1 // G, 0]), n1 // G])


def test_wide_value_heads_reference_moves_midstream():
    """Key norms grow along the sequence, so the running max of every head moves in later
    chunks of a work item (MLA geometry, one split per work item, sampled rows)."""
    B, S1, S2, N1, N2, Dk, Dv, topK = 64, 2, 1024, 128, 1, 576, 512, 512
    g = torch.Generator().manual_seed(11)
    q = torch.randn((B, N1, S1, Dk), generator=g).to(torch.bfloat16)
    ramp = 1.0 + 20.0 * torch.arange(S2, dtype=torch.float32) / S2
    k = (torch.randn((B, N2, S2, Dk), generator=g) * ramp[None, None, :, None]).to(torch.bfloat16)
    v = k[..., :Dv]
    idx = synth.sample_without_replacement(B * S1 * N2, S2, topK, g, sort=True).view(B, S1, N2, topK)
    idx = idx.permute(0, 2, 1, 3).contiguous()
    scale = 1.0 / math.sqrt(Dk)
    log(f"case ramp B={B} S1={S1} S2={S2} N1={N1} Dk={Dk} Dv={Dv} topK={topK}")
    kd = k.to(DEV)
    y, lse = api.sparse_flash_attention(q.to(DEV), kd, kd[..., :Dv], idx.to(DEV), scale, "BNSD", False,
                                        return_lse=True)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(B * S1 * N1, size=512, replace=False))
    g_y, g_lse = oracle.sfa(q, k, v, idx, scale, "BNSD", False, rows=rows)
    yb = y.permute(0, 2, 1, 3).reshape(-1, Dv).float().cpu().numpy()[rows]
    lb = lse.permute(0, 2, 1).reshape(-1).cpu().numpy()[rows]
    rep = precision.gate(yb, g_y, "bf16")
    log(f"  gate: {rep}")
    assert rep["pass"], rep
    np.testing.assert_allclose(lb, g_lse, rtol=2e-6, atol=2e-6)


def test_wide_value_split_partials_in_dirty_reused_workspace():
    """The split partials of the wide-value kernel live in the caller's workspace.  A
    workspace of arbitrary bytes, reused by consecutive calls and by a call of another shape in
    between, gives the oracle's result and the same bits every time."""
    big = synth.SfaShape(B=2, S1=2, S2=3000, N1=128, N2=1, Dk=576, Dv=512, topK=1500, dtype="bf16",
                         layout="BNSD", causal=True, sorted_indices=True)
    small = synth.SfaShape(B=1, S1=1, S2=900, N1=64, N2=1, Dk=576, Dv=512, topK=700, dtype="bf16",
                           layout="BNSD", causal=False)
    ib, isml = synth.sfa_inputs(big, 5), synth.sfa_inputs(small, 6)
    qb, kb, vb, xb = to_dev(ib)
    qs, ks, vs, xs = to_dev(isml)
    need = api.workspace_bytes(qb, kb, vb, xb, big.layout, big.causal)
    need_s = api.workspace_bytes(qs, ks, vs, xs, small.layout, small.causal)
    assert need > 0 and need_s > 0  # both split their index lists
    log(f"case dirty workspace: {need} bytes, shapes {big} / {small}")
    g = torch.Generator().manual_seed(7)
    ws = torch.randint(0, 256, (max(need, need_s),), generator=g, dtype=torch.uint8).to(DEV)
    outs = []
    for i in range(3):
        y, lse = api.sparse_flash_attention(qb, kb, vb, xb, big.scale_value, big.layout, big.causal,
                                            return_lse=True, workspace=ws)
        outs.append((y.clone(), lse.clone()))
        ys = api.sparse_flash_attention(qs, ks, vs, xs, small.scale_value, small.layout, small.causal,
                                        workspace=ws)
        if i == 1:
            ws.fill_(255)
    torch.cuda.synchronize()
    for y, lse in outs[1:]:
        assert torch.equal(y.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse, outs[0][1])
    rows = np.sort(np.random.default_rng(4).choice(big.B * big.S1 * big.N1, size=256, replace=False))
    g_y, g_lse = oracle.sfa(ib["q"], ib["k"], ib["v"], ib["idx"], big.scale_value, big.layout, big.causal, rows=rows)
    yb = gpu_rows_bsnd(outs[0][0], big.layout).reshape(-1, big.Dv).float().cpu().numpy()[rows]
    rep = precision.gate(yb, g_y, "bf16")
    log(f"  gate: {rep}")
    assert rep["pass"], rep
    g_ys, _ = oracle.sfa(isml["q"], isml["k"], isml["v"], isml["idx"], small.scale_value, small.layout,
                         small.causal)
    rep_s = precision.gate(gpu_rows_bsnd(ys, small.layout).reshape(-1, small.Dv).float().cpu().numpy(), g_ys,
                           "bf16")
    log(f"  gate (other shape): {rep_s}")
    assert rep_s["pass"], rep_s


# Decode-like shapes at scale: value = key, few heads per index list, at least 256 index lists
# (one workgroup per list fills the chip), ragged topK, causal with several query rows.
DEC = [
    # (B, S1, S2, N1, N2, D, topK, dtype, layout, causal)
    (32, 1, 8192, 32, 8, 128, 1024, "bf16", "BSND", False),   # the GQA decode geometry, B = 32
    (64, 2, 3000, 8, 2, 128, 1000, "fp16", "BSND", True),     # G = 4, causal with S1 = 2, ragged topK
    (16, 4, 700, 12, 4, 64, 333, "bf16", "BNSD", True),       # G = 3, D = 64
    (128, 1, 5000, 2, 2, 128, 77, "fp16", "BNSD", False),     # G = 1, topK below one round
    (8, 8, 9000, 8, 4, 128, 4100, "bf16", "BSND", True),      # G = 2, long lists, causal S1 = 8
]


@pytest.mark.parametrize("case", DEC, ids=[f"d{i}" for i in range(len(DEC))])
def test_decode_shapes_full_parity(case):
    B, S1, S2, N1, N2, D, topK, dt, layout, causal = case
    shape = synth.SfaShape(B=B, S1=S1, S2=S2, N1=N1, N2=N2, Dk=D, Dv=D, topK=topK, dtype=dt, layout=layout,
                           causal=causal)
    assert B * S1 * N2 >= 256
    run_and_compare(shape, seed=21)


# Decode-like launches (one workgroup of four 32-slot parts per index list, plus four waves that
# only gather) for the other head-dim pairs that take that form: Dv < Dk as a prefix view of K,
# Dk = Dv = 192, and a value tensor of its own.
DEC_DIMS = [
    # (B, S1, S2, N1, N2, Dk, Dv, topK, dtype, layout, causal, value)
    (32, 1, 4096, 32, 8, 192, 128, 512, "fp16", "BSND", False, "alias"),
    (16, 2, 3000, 16, 4, 192, 192, 700, "bf16", "BNSD", True, "alias"),
    (64, 1, 2000, 16, 4, 64, 64, 300, "fp16", "BSND", False, "separate"),
]


@pytest.mark.parametrize("case", DEC_DIMS, ids=[f"dd{i}" for i in range(len(DEC_DIMS))])
def test_decode_head_dim_pairs_full_parity(case):
    B, S1, S2, N1, N2, Dk, Dv, topK, dt, layout, causal, value = case
    shape = synth.SfaShape(B=B, S1=S1, S2=S2, N1=N1, N2=N2, Dk=Dk, Dv=Dv, topK=topK, dtype=dt, layout=layout,
                           causal=causal, value=value)
    assert B * S1 * N2 >= 128
    run_and_compare(shape, seed=23)


def test_decode_shape_masked_rows_and_out_of_range():
    """All-masked rows give +0 and lse = -inf, out-of-range indices are masked, and a row whose
    only unmasked slot is one index gives v[idx] exactly (a decode-like shape at scale)."""
    B, S1, S2, N1, N2, D, topK = 64, 2, 600, 8, 2, 128, 200
    shape = synth.SfaShape(B=B, S1=S1, S2=S2, N1=N1, N2=N2, Dk=D, Dv=D, topK=topK, dtype="bf16",
                           layout="BSND", causal=True)
    inp = synth.sfa_inputs(shape, 8)
    idx = inp["idx"].clone()
    limit = S2 - S1  # row s1 keeps indices <= s1 + S2 - S1
    idx[0, 0, 0, :] = limit + 1 + torch.arange(topK, dtype=torch.int32) % (S2 - limit - 1)  # all masked
    idx[1, 1, 1, :] = S2 + 5                       # all out of range
    idx[2, 0, 0, :] = -3
    idx[2, 0, 0, 17] = 42                          # a single survivor
    idx[3, 1, 0, ::3] = -1                         # a third of the slots out of range
    inp["idx"] = idx
    log(f"case decode masked rows {shape}")
    q, k, v, di = to_dev(inp)
    y, lse = api.sparse_flash_attention(q, k, v, di, shape.scale_value, "BSND", True, return_lse=True)
    torch.cuda.synchronize()
    G = N1 // N2
    y0 = y[0, 0, 0:G].float().cpu()
    assert torch.all(y0 == 0) and not torch.any(torch.signbit(y0))
    assert torch.all(torch.isneginf(lse[0, 0, 0:G].cpu()))
    assert torch.all(y[1, 1, G:2 * G].float().cpu() == 0) and torch.all(torch.isneginf(lse[1, 1, G:2 * G].cpu()))
    assert torch.equal(y[2, 0, 0:G].cpu(), inp["k"][2, 42, 0].unsqueeze(0).expand(G, D))
    # the oracle is not defined for out-of-range indices: compare that row with the problem
    # whose index list holds only its in-range slots
    keep = idx[3, 1, 0] >= 0
    sub = synth.SfaShape(B=1, S1=1, S2=S2, N1=G, N2=1, Dk=D, Dv=D, topK=int(keep.sum()), dtype="bf16",
                         layout="BSND", causal=False)
    q1 = inp["q"][3:4, 1:2, 0:G]
    k1 = inp["k"][3:4, :, 0:1]
    i1 = idx[3:4, 1:2, 0:1, keep]
    g1, _ = oracle.sfa(q1, k1, k1, i1.contiguous(), sub.scale_value, "BSND", False)
    rep = precision.gate(y[3, 1, 0:G].float().cpu().numpy(), g1, "bf16")
    assert rep["pass"], rep


def test_layouts_agree_bitwise_and_copy_meets_gate():
    s = synth.SfaShape(B=2, S1=3, S2=300, N1=16, N2=2, Dk=192, Dv=128, topK=100, dtype="fp16", layout="BSND",
                       causal=True)
    inp = synth.sfa_inputs(s, seed=5)
    q, k, v, idx = to_dev(inp)
    y1 = api.sparse_flash_attention(q, k, v, idx, s.scale_value, "BSND", True)
    # value as an independent copy of the prefix: the separate-value kernels stage twice the
    # bytes per slot, so here they take another chunk length than the aliased ones (see the
    # bitwise test below for shapes where both take the same)
    y2 = api.sparse_flash_attention(q, k, v.contiguous(), idx, s.scale_value, "BSND", True)
    p = lambda t: t.permute(0, 2, 1, 3).contiguous()
    kp = p(k)
    y3 = api.sparse_flash_attention(p(q), kp, kp[..., :128], p(idx), s.scale_value, "BNSD", True)
    torch.cuda.synchronize()
    # same per-element arithmetic in both layouts: identical bits
    same = torch.equal(y1, y3.permute(0, 2, 1, 3))
    assert same, "BSND and BNSD results differ"
    g, _ = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], s.scale_value, "BSND", True)
    for y in (y1, y2):
        assert precision.gate(y.reshape(-1, 128).float().cpu().numpy(), g, "fp16")["pass"]


@pytest.mark.parametrize("B,S1,N1,N2,Dk,Dv,topK,dtype,causal", [
    (2, 2, 4, 1, 64, 64, 333, "fp16", False),     # 16-wide tiles, 4 slot parts, 3 splits + merge
    (4, 4, 64, 1, 128, 128, 256, "bf16", True),   # 32-wide tiles x 2, 2 slot parts, 4 splits
    (1, 4, 32, 1, 512, 512, 256, "bf16", False),  # 16-wide tiles x 2, wide values, 8 splits
])
def test_alias_and_copy_agree_bitwise(B, S1, N1, N2, Dk, Dv, topK, dtype, causal):
    """Value given as key itself (one gather serves both) and as a separate copy with the same
    values: on these shapes both kernels take the same head tiling, chunk length and split (on a
    256-CU MI355X), so every product and sum is the same and the outputs are bitwise equal."""
    s = synth.SfaShape(B=B, S1=S1, S2=1024, N1=N1, N2=N2, Dk=Dk, Dv=Dv, topK=topK, dtype=dtype,
                       layout="BSND", causal=causal, value="alias")
    log(f"alias vs copy {s}")
    inp = synth.sfa_inputs(s, seed=21)
    q, k, v, idx = to_dev(inp)
    assert v.data_ptr() == k.data_ptr()
    y1, l1 = api.sparse_flash_attention(q, k, v, idx, s.scale_value, "BSND", causal, return_lse=True)
    vc = k.clone()
    y2, l2 = api.sparse_flash_attention(q, k, vc, idx, s.scale_value, "BSND", causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), f"max |diff| {(y1.float() - y2.float()).abs().max().item()}"
    assert torch.equal(l1, l2)
    g, _ = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], s.scale_value, "BSND", causal)
    assert precision.gate(y1.reshape(-1, Dv).float().cpu().numpy(), g, dtype)["pass"]


def test_permuted_indices_within_tolerance():
    s = synth.SfaShape(B=1, S1=2, S2=1000, N1=8, N2=1, Dk=128, Dv=128, topK=256, dtype="bf16")
    inp = synth.sfa_inputs(s, seed=9)
    q, k, v, idx = to_dev(inp)
    perm = torch.randperm(s.topK, generator=torch.Generator().manual_seed(1)).to(DEV)
    y1 = api.sparse_flash_attention(q, k, v, idx, s.scale_value)
    y2 = api.sparse_flash_attention(q, k, v, idx[..., perm].contiguous(), s.scale_value)
    g, _ = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], s.scale_value)
    for y in (y1, y2):
        assert precision.gate(y.reshape(-1, 128).float().cpu().numpy(), g, "bf16")["pass"]


def test_out_of_range_indices_are_masked_not_read():
    B, S1, S2, N1, N2, D = 1, 2, 16, 4, 1, 64
    q, k, v, _ = _custom(B, S1, S2, N1, N2, D, None)
    idx = torch.tensor([[[[3, -1, 16, 1 << 30]], [[-5, 5, 99, 16]]]], dtype=torch.int32)
    y = api.sparse_flash_attention(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), 0.2, "BSND", False).cpu()
    for n1 in range(N1):
        assert torch.equal(y[0, 0, n1], v[0, 3, 0])
        assert torch.equal(y[0, 1, n1], v[0, 5, 0])


def test_empty_batch():
    s = synth.SfaShape(B=1, S1=1, S2=64, N1=4, N2=1, Dk=64, Dv=64, topK=16)
    q = torch.empty((0, 1, 4, 64), dtype=torch.float16, device=DEV)
    k = torch.empty((0, 64, 1, 64), dtype=torch.float16, device=DEV)
    idx = torch.empty((0, 1, 1, 16), dtype=torch.int32, device=DEV)
    y = api.sparse_flash_attention(q, k, k, idx, 0.125)
    assert y.shape == (0, 1, 4, 64)
