"""GPU parity of the block-sparse (BSR) attention kernel against the fp64 oracle."""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import precision
from sparse_attention_13_amd import api, synth
from tests.conftest import golden_path

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_bsr(q, k, v, indptr, indices, M, N, R, C, causal=False, sm_scale=None, rows=None, dtype="fp16", tag="",
            mask=None):
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    log(f"bsr case {tag} M={M} N={N} R={R} C={C} Hq={Hq} Hkv={Hkv} D={D} causal={causal} nnz={len(indices)} "
        f"mask={'none' if mask is None else 'given'}")
    w = api.BlockSparseAttentionWrapper()
    w.plan(indptr, indices, M, N, R, C, Hq, Hkv, D, mask=mask, causal=causal, sm_scale=sm_scale,
           q_data_type=q.dtype)
    o, lse = w.run(q.to(DEV), k.to(DEV), v.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    yb = o.reshape(-1, D).float().cpu().numpy()
    lb = lse.reshape(-1).cpu().numpy()
    g_y, g_lse = oracle.bsr(q, k, v, indptr, indices, R, C, causal=causal, sm_scale=sm_scale, rows=rows, mask=mask)
    if rows is not None:
        yb, lb = yb[rows], lb[rows]
    rep = precision.gate(yb, g_y, dtype)
    log(f"  gate: {rep}")
    if os.environ.get("SFA_PARITY_LOG"):
        with open(os.environ["SFA_PARITY_LOG"], "a") as f:
            f.write(json.dumps({"case": f"bsr {tag} M={M} N={N} R={R} C={C} Hq={Hq} Hkv={Hkv} D={D} causal={causal}",
                                **rep}) + "\n")
    assert rep["pass"], rep
    fin = np.isfinite(g_lse)
    assert np.array_equal(np.isfinite(lb), fin)
    np.testing.assert_allclose(lb[fin], g_lse[fin], rtol=2e-6, atol=2e-6)
    if (~fin).any():
        assert np.all(yb[~fin] == 0.0)
    return rep


def _rand(shape, seed, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def test_page_worked_example():
    ex = json.load(open(golden_path("bsr_worked_example.json")))
    M, N, R, C = ex["M"], ex["N"], ex["R"], ex["C"]
    Hq, Hkv, D = ex["num_qo_heads"], ex["num_kv_heads"], ex["head_dim"]
    q, k, v = _rand((M, Hq, D), 1), _rand((N, Hkv, D), 2), _rand((N, Hkv, D), 3)
    run_bsr(q, k, v, ex["indptr"], ex["indices"], M, N, R, C, tag="page-example")


def _pattern(MB, NB, per_row, seed, empty_rows=()):
    g = torch.Generator().manual_seed(seed)
    indptr, indices = [0], []
    for br in range(MB):
        cols = [] if br in empty_rows else sorted(torch.randperm(NB, generator=g)[:per_row].tolist())
        indices += cols
        indptr.append(len(indices))
    return indptr, indices


@pytest.mark.parametrize("M,N,R,C,Hq,Hkv,D,per_row,causal,dt", [
    (128, 128, 16, 16, 8, 2, 128, 3, False, "fp16"),
    (37, 64, 4, 8, 4, 1, 64, 5, False, "fp16"),      # ragged last block row, C not a multiple of 32
    (1024, 1024, 64, 64, 32, 8, 128, 4, False, "fp16"),
    (200, 256, 8, 32, 16, 16, 128, 3, True, "bf16"),  # causal, G = 1
    (96, 96, 32, 1, 6, 2, 256, 40, False, "bf16"),    # column blocks of one key, D = 256
    (64, 80, 16, 16, 4, 4, 64, 5, True, "fp16"),      # M < N, causal
])
def test_small_patterns(M, N, R, C, Hq, Hkv, D, per_row, causal, dt):
    tdt = torch.float16 if dt == "fp16" else torch.bfloat16
    MB, NB = (M + R - 1) // R, N // C
    indptr, indices = _pattern(MB, NB, min(per_row, NB), seed=M + N, empty_rows=(1,))
    q, k, v = _rand((M, Hq, D), 4, tdt), _rand((N, Hkv, D), 5, tdt), _rand((N, Hkv, D), 6, tdt)
    run_bsr(q, k, v, indptr, indices, M, N, R, C, causal=causal, dtype=dt, tag="small")



@pytest.mark.parametrize("D,causal,masked,dt", [
    (128, False, False, "fp16"),
    (128, True, False, "bf16"),
    (128, False, True, "fp16"),
    (64, False, False, "bf16"),
    (64, True, True, "fp16"),
])
def test_eight_wave_workgroups(D, causal, masked, dt):
    """64-row blocks of 4 query heads per KV head: 256 query vectors per block row, eight waves per
    workgroup (two per SIMD), one workgroup per (block row, KV head) and every list whole.  Block
    row br keeps br % 10 column blocks of 32 keys, so the launch holds work items of 0 to 9 ring
    chunks: the ring's first steps, its steady state and its drain."""
    M, R, C, Hq, Hkv = 64 * 40, 64, 32, 32, 8
    N = M if causal else 32 * 12
    tdt = torch.float16 if dt == "fp16" else torch.bfloat16
    MB, NB = M // R, N // C
    g = torch.Generator().manual_seed(D + 2 * causal + masked)
    indptr, indices = [0], []
    for br in range(MB):
        n = br % 10
        if causal:  # blocks at or left of the diagonal
            cols = sorted(torch.randperm(br * 2 + 2, generator=g)[:n].tolist())
        else:
            cols = sorted(torch.randperm(NB, generator=g)[:n].tolist())
        indices += cols
        indptr.append(len(indices))
    mask = None
    if masked:
        mask = torch.rand((len(indices), R, C), generator=g) < 0.6
    q, k, v = _rand((M, Hq, D), 21, tdt), _rand((N, Hkv, D), 22, tdt), _rand((N, Hkv, D), 23, tdt)
    rows = np.arange(0, M * Hq, 5)  # every block row and head
    run_bsr(q, k, v, indptr, indices, M, N, R, C, causal=causal, dtype=dt, rows=rows, tag="eight waves",
            mask=mask)

def test_workload_at_full_size():
    s = synth.WORKLOADS["bsr"]
    inp = synth.bsr_inputs(s, seed=0)
    nrows = s.M * s.Hq
    rows = np.sort(np.random.default_rng(11).choice(nrows, size=1024, replace=False))
    run_bsr(inp["q"], inp["k"], inp["v"], inp["indptr"], inp["indices"], s.M, s.N, s.R, s.C, rows=rows,
            tag="workload")


@pytest.mark.parametrize("M,N,R,C,Hq,Hkv,D,per_row,causal,dt,density", [
    (128, 128, 16, 16, 8, 2, 128, 3, False, "fp16", 0.5),
    (37, 64, 4, 8, 4, 1, 64, 5, False, "fp16", 0.3),    # ragged last block row; 8-key blocks share chunks
    (200, 256, 8, 32, 16, 16, 128, 3, True, "bf16", 0.6),  # causal is ignored with a mask
    (96, 96, 32, 1, 6, 2, 256, 40, False, "bf16", 0.5),   # 1-key column blocks
    (256, 512, 64, 64, 32, 8, 128, 4, False, "fp16", 0.7),  # the workload's block and head shape
])
def test_block_mask(M, N, R, C, Hq, Hkv, D, per_row, causal, dt, density):
    """Per-block mask [nnz, R, C] of the plan page (NEXT row of the block-sparse path); some query
    rows lose every key (they output zeros, lse = -inf)."""
    tdt = torch.float16 if dt == "fp16" else torch.bfloat16
    MB, NB = (M + R - 1) // R, N // C
    indptr, indices = _pattern(MB, NB, min(per_row, NB), seed=M + 2 * N, empty_rows=(1,))
    g = torch.Generator().manual_seed(M + N + R)
    mask = torch.rand((len(indices), R, C), generator=g) < density
    if MB > 2:
        mask[indptr[2]:indptr[3], R // 2] = False  # one query row of block row 2 keeps no key
    q, k, v = _rand((M, Hq, D), 7, tdt), _rand((N, Hkv, D), 8, tdt), _rand((N, Hkv, D), 9, tdt)
    run_bsr(q, k, v, indptr, indices, M, N, R, C, causal=causal, dtype=dt, tag="mask", mask=mask)


def test_all_true_mask_is_bitwise_unmasked():
    M, N, R, C, Hq, Hkv, D = 128, 256, 16, 32, 8, 2, 128
    indptr, indices = _pattern(M // R, N // C, 3, seed=3)
    q, k, v = _rand((M, Hq, D), 1).to(DEV), _rand((N, Hkv, D), 2).to(DEV), _rand((N, Hkv, D), 3).to(DEV)
    outs = []
    for mask in (None, torch.ones((len(indices), R, C), dtype=torch.bool)):
        w = api.BlockSparseAttentionWrapper()
        w.plan(indptr, indices, M, N, R, C, Hq, Hkv, D, mask=mask)
        outs.append(w.run(q, k, v))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_plan_rejects_bad_patterns():
    w = api.BlockSparseAttentionWrapper()
    from sparse_attention_13_amd import binding
    with pytest.raises(binding.SfaError):
        w.plan([0, 2, 3], [0, 0, 1], 4, 4, 2, 2, 4, 2, 64)  # repeated column block in a row
    with pytest.raises(binding.SfaError):
        w.plan([0, 1, 2], [0, 5], 4, 4, 2, 2, 4, 2, 64)  # column block out of range
    with pytest.raises(binding.SfaError):
        w.run(torch.zeros(1, device=DEV), torch.zeros(1, device=DEV), torch.zeros(1, device=DEV))  # run before plan


def test_user_float_workspace_holds_the_split_partials():
    # One long block row per KV head: the plan splits each key list, so the runs write their split
    # partials into the caller's float workspace (128 MB, as the page recommends).
    M, N, R, C, Hq, Hkv, D = 16, 4096, 16, 64, 8, 2, 128
    indptr, indices = [0, 64], list(range(64))
    q, k, v = _rand((M, Hq, D), 31), _rand((N, Hkv, D), 32), _rand((N, Hkv, D), 33)
    fws = torch.full((128 << 20,), 0x7F, dtype=torch.uint8, device=DEV)  # a sentinel byte pattern
    w = api.BlockSparseAttentionWrapper(fws)
    w.plan(indptr, indices, M, N, R, C, Hq, Hkv, D)
    assert w._bufs.float_ws is fws
    o, lse = w.run(q.to(DEV), k.to(DEV), v.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    head = fws[: 1 << 20]
    assert int((head != 0x7F).sum()) > 0, "the float workspace was not written"
    g_y, g_lse = oracle.bsr(q, k, v, indptr, indices, R, C)
    rep = precision.gate(o.reshape(-1, D).float().cpu().numpy(), g_y, "fp16")
    log(f"  gate: {rep}")
    assert rep["pass"], rep
    # a buffer smaller than the plan needs is refused before anything runs
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    w2 = api.BlockSparseAttentionWrapper(small)
    with pytest.raises(Exception) as e:
        w2.plan(indptr, indices, M, N, R, C, Hq, Hkv, D)
    assert "WORKSPACE" in str(e.value)
    # the same float workspace serves a second wrapper whose runs do not overlap the first's
    w3 = api.BlockSparseAttentionWrapper(fws)
    w3.plan(indptr, indices, M, N, R, C, Hq, Hkv, D)
    o3 = w3.run(q.to(DEV), k.to(DEV), v.to(DEV))
    o1 = w.run(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o) and torch.equal(o3, o)
