"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

None of these re-types the oracle's loop: each compares it with a library routine
(torch's scaled_dot_product_attention / logsumexp in fp64), a closed form, an
invariant, a printed worked example, or a second formulation of the operator.
"""
import json
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from sparse_attention_13_amd import synth
from tests.conftest import golden_path

torch.set_num_threads(4)


def _sdpa(q, k, v, bias, scale):
    """torch SDPA in fp64.  q [Hq, L, E], k [Hkv, S, E], v [Hkv, S, Ev], bias [Hq or 1, L, S]."""
    G = q.shape[0] // k.shape[0]
    kk = k.repeat_interleave(G, dim=0)  # query head h reads KV head h // G
    vv = v.repeat_interleave(G, dim=0)
    return F.scaled_dot_product_attention(q[None], kk[None], vv[None], attn_mask=bias[None], scale=scale)[0]


def _bias_from_bool(mask):
    b = torch.zeros(mask.shape, dtype=torch.float64)
    b[~mask] = -math.inf
    return b


def _rand(shape, seed, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


# ---------------------------------------------------------------- dense masked


@pytest.mark.parametrize("Hq,Hkv,D,Dv", [(8, 2, 32, 16), (4, 4, 64, 64), (6, 1, 16, 32)])
def test_dense_masked_matches_sdpa(Hq, Hkv, D, Dv):
    qo, kv = 7, 23
    q, k, v = _rand((qo, Hq, D), 1), _rand((kv, Hkv, D), 2), _rand((kv, Hkv, Dv), 3)
    g = torch.Generator().manual_seed(4)
    mask = torch.rand((qo, kv), generator=g) < 0.4
    mask[:, 5] = True  # every row keeps at least one key
    scale = 0.37
    y, lse = oracle.dense_masked(q, k, v, mask=mask, scale=scale)
    ref = _sdpa(q.double().transpose(0, 1), k.double().transpose(0, 1), v.double().transpose(0, 1),
                _bias_from_bool(mask)[None].expand(Hq, qo, kv), scale)  # [Hq, qo, Dv]
    np.testing.assert_allclose(y.reshape(qo, Hq, Dv), ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)
    # LSE: log-sum-exp of the scaled logits over the allowed keys (library logsumexp)
    G = Hq // Hkv
    kk = k.double().repeat_interleave(G, dim=1)
    logits = torch.einsum("qhd,khd->qhk", q.double(), kk) * scale
    logits = logits.masked_fill(~mask[:, None, :], -math.inf)
    np.testing.assert_allclose(lse.reshape(qo, Hq), torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_dense_causal_page_example():
    """single_prefill_with_kv_cache page: causal=True equals the tril(diagonal=kv_len-qo_len) custom mask."""
    ex = json.load(open(golden_path("dense_causal_example.json")))
    qo, kv, Hq, Hkv, D = ex["qo_len"], ex["kv_len"], ex["num_qo_heads"], ex["num_kv_heads"], ex["head_dim"]
    q, k, v = _rand((qo, Hq, D), 11), _rand((kv, Hkv, D), 12), _rand((kv, Hkv, D), 13)
    rows = list(range(0, qo * Hq, 37))  # a spread of (row, head) pairs
    y_c, lse_c = oracle.dense_masked(q, k, v, causal=True, rows=rows)
    mask = torch.tril(torch.ones((qo, kv), dtype=torch.bool), diagonal=kv - qo)
    y_m, lse_m = oracle.dense_masked(q, k, v, mask=mask, rows=rows)
    assert np.array_equal(y_c, y_m) and np.array_equal(lse_c, lse_m)
    # and both equal the library routine with that mask on a few query rows
    sel = [0, 1, 63, 127]
    ref = _sdpa(q[sel].double().transpose(0, 1), k.double().transpose(0, 1), v.double().transpose(0, 1),
                _bias_from_bool(mask[sel])[None].expand(Hq, len(sel), kv), 1.0 / math.sqrt(D))
    y_all, _ = oracle.dense_masked(q, k, v, causal=True, rows=[r * Hq + h for r in sel for h in range(Hq)])
    np.testing.assert_allclose(y_all.reshape(len(sel), Hq, D), ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)
    assert list(ex["output_shape"]) == [qo, Hq, D]


# ---------------------------------------------------------------- BSR


def test_bsr_page_example():
    """BlockSparseAttentionWrapper page: indptr/indices with 1x1 blocks denote the printed mask,
    and BSR attention equals dense attention under that mask."""
    ex = json.load(open(golden_path("bsr_worked_example.json")))
    M, N, R, C = ex["M"], ex["N"], ex["R"], ex["C"]
    Hq, Hkv, D = ex["num_qo_heads"], ex["num_kv_heads"], ex["head_dim"]
    mask = oracle.bsr_mask(ex["indptr"], ex["indices"], M, N, R, C)
    assert np.array_equal(mask, np.array(ex["mask"], dtype=bool))
    q, k, v = _rand((M, Hq, D), 21), _rand((N, Hkv, D), 22), _rand((N, Hkv, D), 23)
    y_b, lse_b = oracle.bsr(q, k, v, ex["indptr"], ex["indices"], R, C)
    y_d, lse_d = oracle.dense_masked(q, k, v, mask=torch.tensor(ex["mask"], dtype=torch.bool))
    assert np.array_equal(y_b, y_d) and np.array_equal(lse_b, lse_d)
    ref = _sdpa(q.double().transpose(0, 1), k.double().transpose(0, 1), v.double().transpose(0, 1),
                _bias_from_bool(torch.tensor(ex["mask"], dtype=torch.bool))[None].expand(Hq, M, N),
                1.0 / math.sqrt(D))
    np.testing.assert_allclose(y_b.reshape(M, Hq, D), ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)


def test_bsr_mask_blocks_and_ragged_last_row():
    # M not a multiple of R: the last block row is partial (MB = ceil(M / R))
    M, N, R, C = 10, 12, 4, 3
    indptr = [0, 2, 3, 5]
    indices = [0, 3, 1, 2, 3]
    mask = oracle.bsr_mask(indptr, indices, M, N, R, C)
    expect = np.zeros((M, N), dtype=bool)
    for br, cols in enumerate([[0, 3], [1], [2, 3]]):
        for c in cols:
            expect[br * R: min(M, (br + 1) * R), c * C:(c + 1) * C] = True
    assert np.array_equal(mask, expect)
    with pytest.raises(ValueError):
        oracle.bsr_mask([0, 1, 2, 3], [0, 1, 4], M, N, R, C)  # column block out of range


def test_bsr_equals_topk_with_row_lists():
    """BSR with 1x1 blocks is the top-K operator with each row's column list as its indices."""
    M = N = 16
    Hq, Hkv, D = 4, 2, 64
    g = torch.Generator().manual_seed(5)
    per_row = 5
    cols = [sorted(torch.randperm(N, generator=g)[:per_row].tolist()) for _ in range(M)]
    indptr = [0]
    for c in cols:
        indptr.append(indptr[-1] + len(c))
    indices = [c for row in cols for c in row]
    q, k, v = _rand((M, Hq, D), 31), _rand((N, Hkv, D), 32), _rand((N, Hkv, D), 33)
    y_b, lse_b = oracle.bsr(q, k, v, indptr, indices, 1, 1, sm_scale=0.2)
    idx = torch.tensor(cols, dtype=torch.int32).view(1, M, 1, per_row).expand(1, M, Hkv, per_row).contiguous()
    y_s, lse_s = oracle.sfa(q[None], k[None], v[None], idx, 0.2, layout="BSND")
    np.testing.assert_allclose(y_s, y_b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse_s, lse_b, rtol=1e-13, atol=1e-14)


def _block_pattern(MB, NB, per_row, seed):
    g = torch.Generator().manual_seed(seed)
    indptr, indices = [0], []
    for _ in range(MB):
        cols = sorted(torch.randperm(NB, generator=g)[:per_row].tolist())
        indices += cols
        indptr.append(len(indices))
    return indptr, indices


def test_bsr_block_mask_matches_sdpa():
    """Per-block mask [nnz, R, C] of the plan page: element (i, j) of stored block t masks query
    row br*R + i against key indices[t]*C + j.  The dense bias is built here block by block and
    fed to torch SDPA in fp64; rows with no allowed key give 0 and lse = -inf."""
    M, N, R, C = 22, 24, 8, 4          # ragged last block row (22 = 2*8 + 6)
    Hq, Hkv, D = 4, 2, 32
    MB, NB = (M + R - 1) // R, N // C
    indptr, indices = _block_pattern(MB, NB, 3, 41)
    nnz = indptr[-1]
    g = torch.Generator().manual_seed(42)
    bmask = torch.rand((nnz, R, C), generator=g) < 0.5
    bmask[0] = False                   # one fully masked block
    bmask[indptr[1]:indptr[2], 3] = False  # row 8 + 3 loses every key of its block row
    q, k, v = _rand((M, Hq, D), 43), _rand((N, Hkv, D), 44), _rand((N, Hkv, D), 45)
    y, lse = oracle.bsr(q, k, v, indptr, indices, R, C, sm_scale=0.3, mask=bmask)
    dense = torch.zeros((M, N), dtype=torch.bool)
    for br in range(MB):
        for t in range(indptr[br], indptr[br + 1]):
            for i in range(R):
                if br * R + i < M:
                    dense[br * R + i, indices[t] * C:(indices[t] + 1) * C] = bmask[t, i]
    assert not dense[R + 3].any()
    ref = _sdpa(q.double().transpose(0, 1), k.double().transpose(0, 1), v.double().transpose(0, 1),
                _bias_from_bool(dense)[None].expand(Hq, M, N), 0.3).transpose(0, 1).numpy()  # [M, Hq, D]
    alive = dense.any(dim=1).numpy()
    y = y.reshape(M, Hq, D)
    lse = lse.reshape(M, Hq)
    np.testing.assert_allclose(y[alive], ref[alive], rtol=1e-12, atol=1e-13)
    assert np.all(y[~alive] == 0.0) and np.all(np.isneginf(lse[~alive])) and np.all(np.isfinite(lse[alive]))


def test_bsr_block_mask_special_cases():
    M, N, R, C = 16, 16, 4, 4
    Hq, Hkv, D = 2, 1, 16
    indptr, indices = _block_pattern(4, 4, 2, 51)
    q, k, v = _rand((M, Hq, D), 52), _rand((N, Hkv, D), 53), _rand((N, Hkv, D), 54)
    y0, l0 = oracle.bsr(q, k, v, indptr, indices, R, C)
    # all-true mask = no mask
    y1, l1 = oracle.bsr(q, k, v, indptr, indices, R, C, mask=torch.ones((indptr[-1], R, C), dtype=torch.bool))
    assert np.array_equal(y0, y1) and np.array_equal(l0, l1)
    # with a mask the causal flag is ignored (plan page)
    g = torch.Generator().manual_seed(55)
    bm = torch.rand((indptr[-1], R, C), generator=g) < 0.6
    ya, la = oracle.bsr(q, k, v, indptr, indices, R, C, mask=bm)
    yb, lb = oracle.bsr(q, k, v, indptr, indices, R, C, mask=bm, causal=True)
    assert np.array_equal(ya, yb) and np.array_equal(la, lb)
    # 1x1 blocks: a False block is the same as leaving the block out of the pattern
    M1 = N1 = 12
    ip1, ix1 = _block_pattern(M1, N1, 5, 56)
    keep = torch.rand((ip1[-1],), generator=g) < 0.7
    q1, k1, v1 = _rand((M1, Hq, D), 57), _rand((N1, Hkv, D), 58), _rand((N1, Hkv, D), 59)
    ym, lm = oracle.bsr(q1, k1, v1, ip1, ix1, 1, 1, mask=keep.view(-1, 1, 1))
    ip2, ix2 = [0], []
    for br in range(M1):
        for t in range(ip1[br], ip1[br + 1]):
            if keep[t]:
                ix2.append(ix1[t])
        ip2.append(len(ix2))
    yd, ld = oracle.bsr(q1, k1, v1, ip2, ix2, 1, 1)
    assert np.array_equal(ym, yd) and np.array_equal(lm, ld)


# ---------------------------------------------------------------- variable block-sparse


def _vb_mask_by_lookup(bmap, rs, cs):
    """Element-by-element mask of a variable block pattern: row r lies in the block row i with
    cum_rows[i] <= r < cum_rows[i + 1] (found by bisection; empty blocks are skipped)."""
    import bisect
    bmap, rs, cs = np.asarray(bmap, dtype=bool), np.asarray(rs), np.asarray(cs)
    out = []
    for h in range(bmap.shape[0]):
        cr = np.concatenate([[0], np.cumsum(rs[h])]).tolist()
        cc = np.concatenate([[0], np.cumsum(cs[h])]).tolist()
        m = np.zeros((cr[-1], cc[-1]), dtype=bool)
        for r in range(cr[-1]):
            i = bisect.bisect_right(cr, r) - 1
            for c in range(cc[-1]):
                m[r, c] = bmap[h, i, bisect.bisect_right(cc, c) - 1]
        out.append(m)
    return np.stack(out)


def test_vbsr_page_example_mask_and_output():
    ex = json.load(open(golden_path("variable_block_example.json")))
    want = np.array(ex["dense_mask_derived_by_hand"]["mask"], dtype=bool)
    got = oracle.variable_block_mask(ex["block_mask_map"], ex["block_row_sz"], ex["block_col_sz"])
    assert got.shape == (1, 6, 6) and np.array_equal(got[0], want)
    assert np.array_equal(_vb_mask_by_lookup(ex["block_mask_map"], ex["block_row_sz"], ex["block_col_sz"])[0], want)
    L, D = ex["seq_len"], ex["head_dim"]
    q, k, v = _rand((1, L, D), 61), _rand((1, L, D), 62), _rand((1, L, D), 63)
    y, lse = oracle.vbsr(q, k, v, ex["block_mask_map"], ex["block_row_sz"], ex["block_col_sz"])
    scale = 1.0 / math.sqrt(D)
    bias = _bias_from_bool(torch.from_numpy(want))[None]
    ref = _sdpa(q.double(), k.double(), v.double(), bias, scale)
    np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-12)
    lref = torch.logsumexp(scale * q.double()[0] @ k.double()[0].T + bias[0], dim=-1)
    np.testing.assert_allclose(lse[0], lref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_vbsr_per_head_patterns_match_sdpa(causal):
    """Different sizes and maps per KV head (an empty block row and column, a block row with no
    attended block), GQA with query head n on KV head n // G, M != N for the causal offset."""
    Hkv, G, D = 2, 3, 16
    rs = [[4, 0, 5, 4], [2, 6, 3, 2]]       # M = 13
    cs = [[5, 3, 0, 9], [1, 7, 6, 3]]       # N = 17
    bmap = np.array([[[1, 0, 1, 0], [1, 1, 1, 1], [0, 0, 0, 0], [0, 1, 0, 1]],
                     [[0, 1, 1, 0], [1, 0, 0, 1], [1, 1, 0, 0], [0, 0, 1, 1]]], dtype=bool)
    M, N = 13, 17
    q, k, v = _rand((Hkv * G, M, D), 64), _rand((Hkv, N, D), 65), _rand((Hkv, N, D), 66)
    y, lse = oracle.vbsr(q, k, v, bmap, rs, cs, causal=causal)
    mask = _vb_mask_by_lookup(bmap, rs, cs)
    if causal:
        mask &= np.arange(N)[None, None, :] <= np.arange(M)[None, :, None] + (N - M)
    mq = torch.from_numpy(mask).repeat_interleave(G, dim=0)  # [Hq, M, N]
    scale = 1.0 / math.sqrt(D)
    ref = _sdpa(q.double(), k.double(), v.double(), _bias_from_bool(mq), scale).numpy()
    live = mq.any(dim=-1).numpy()
    assert (~live).any() and live.any()
    np.testing.assert_allclose(y[live], ref[live], rtol=0, atol=1e-12)
    assert np.all(y[~live] == 0.0) and np.all(np.isneginf(lse[~live]))
    s = scale * q.double() @ k.double().repeat_interleave(G, dim=0).transpose(1, 2) + _bias_from_bool(mq)
    np.testing.assert_allclose(lse[live], torch.logsumexp(s, dim=-1).numpy()[live], rtol=0, atol=1e-12)
    # a subset of query rows is the same computation
    sub = [0, 5, 12]
    ys, ls = oracle.vbsr(q, k, v, bmap, rs, cs, causal=causal, qrows=sub)
    assert np.array_equal(ys, y[:, sub]) and np.array_equal(ls, lse[:, sub])


@pytest.mark.parametrize("causal", [False, True])
def test_vbsr_uniform_blocks_equal_bsr(causal):
    """Equal block sizes and the same map on every KV head: the BSR operator (a separate C
    implementation) on the same pattern, after the HND / NHD transposes."""
    M, N, R, C, Hq, Hkv, D = 16, 24, 4, 4, 4, 2, 16
    indptr, indices = _block_pattern(M // R, N // C, 3, 67)
    bm = np.zeros((M // R, N // C), dtype=bool)
    for i in range(M // R):
        bm[i, indices[indptr[i]:indptr[i + 1]]] = True
    q, k, v = _rand((M, Hq, D), 68), _rand((N, Hkv, D), 69), _rand((N, Hkv, D), 70)
    yb, lb = oracle.bsr(q, k, v, indptr, indices, R, C, causal=causal)
    yv, lv = oracle.vbsr(q.permute(1, 0, 2), k.permute(1, 0, 2), v.permute(1, 0, 2), np.stack([bm] * Hkv),
                         [[R] * (M // R)] * Hkv, [[C] * (N // C)] * Hkv, causal=causal)
    np.testing.assert_allclose(yv.transpose(1, 0, 2).reshape(M * Hq, D), yb, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(lv.T.reshape(-1)), np.isfinite(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lv.T.reshape(-1)[fin], lb[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- top-K operator


def _to_layout(t, layout):
    """[B, S, N, D] -> layout order."""
    return t if layout == "BSND" else t.permute(0, 2, 1, 3).contiguous()


def _sfa_via_dense(q, k, v, idx, scale, causal):
    """Second formulation: top-K attention == dense attention over all S2 keys with additive
    bias log(multiplicity of j in the row's index list), -inf where absent or causally masked.
    All tensors BSND.  Returns [B, S1, N1, Dv] (NaN on fully masked rows)."""
    B, S1, N1, Dk = q.shape
    S2, N2 = k.shape[1], k.shape[2]
    G = N1 // N2
    out = torch.empty((B, S1, N1, v.shape[-1]), dtype=torch.float64)
    for b in range(B):
        count = torch.zeros((N2, S1, S2), dtype=torch.float64)
        for s1 in range(S1):
            for n2 in range(N2):
                count[n2, s1].index_add_(0, idx[b, s1, n2].long(), torch.ones(idx.shape[-1], dtype=torch.float64))
        if causal:
            j = torch.arange(S2)[None, :]
            i = torch.arange(S1)[:, None]
            count[:, j.expand(S1, S2) > i + (S2 - S1)] = 0
        bias = torch.log(count).repeat_interleave(G, dim=0)  # [N1, S1, S2], log 0 = -inf
        o = _sdpa(q[b].double().transpose(0, 1), k[b].double().transpose(0, 1), v[b].double().transpose(0, 1),
                  bias, scale)
        out[b] = o.transpose(0, 1)
    return out


@pytest.mark.parametrize("layout", ["BSND", "BNSD"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S1,S2,N1,N2,Dk,Dv,topK", [
    (2, 3, 9, 4, 2, 32, 16, 5),
    (1, 4, 6, 3, 1, 16, 16, 6),
    (1, 2, 40, 8, 1, 64, 32, 17),
])
def test_sfa_matches_dense_with_multiplicity(layout, causal, B, S1, S2, N1, N2, Dk, Dv, topK):
    q, k, v = _rand((B, S1, N1, Dk), 41), _rand((B, S2, N2, Dk), 42), _rand((B, S2, N2, Dv), 43)
    g = torch.Generator().manual_seed(44)
    idx = torch.randint(0, S2, (B, S1, N2, topK), generator=g, dtype=torch.int32)  # duplicates allowed
    scale = 0.3
    ref = _sfa_via_dense(q, k, v, idx, scale, causal)
    y, lse = oracle.sfa(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout),
                        _to_layout(idx, layout), scale, layout=layout, causal=causal)
    y = torch.from_numpy(y).view(B, S1, N1, Dv)
    finite = torch.isfinite(ref).all(dim=-1)
    assert torch.allclose(y[finite], ref[finite], rtol=1e-12, atol=1e-13)
    assert torch.all(y[~finite] == 0)  # rows with no surviving slot output zeros


@pytest.mark.parametrize("causal", [False, True])
def test_sfa_identity_indices_is_dense_attention(causal):
    B, S1, S2, N1, N2, D = 2, 5, 12, 6, 3, 32
    q, k, v = _rand((B, S1, N1, D), 51), _rand((B, S2, N2, D), 52), _rand((B, S2, N2, D), 53)
    idx = torch.arange(S2, dtype=torch.int32).view(1, 1, 1, S2).expand(B, S1, N2, S2).contiguous()
    y, _ = oracle.sfa(q, k, v, idx, 1.0 / math.sqrt(D), causal=causal)
    y = y.reshape(B, S1, N1, D)
    mask = torch.ones((S1, S2), dtype=torch.bool)
    if causal:
        mask = torch.tril(mask, diagonal=S2 - S1)
    for b in range(B):
        ref = _sdpa(q[b].double().transpose(0, 1), k[b].double().transpose(0, 1), v[b].double().transpose(0, 1),
                    _bias_from_bool(mask)[None].expand(N1, S1, S2), 1.0 / math.sqrt(D))
        np.testing.assert_allclose(y[b], ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)


def test_sfa_permutation_invariance():
    B, S1, S2, N1, N2, D, topK = 1, 3, 50, 4, 2, 64, 20
    q, k = _rand((B, S1, N1, D), 61), _rand((B, S2, N2, D), 62)
    idx = synth.sample_without_replacement(B * S1 * N2, S2, topK, torch.Generator().manual_seed(63)).view(B, S1, N2, topK)
    perm = torch.randperm(topK, generator=torch.Generator().manual_seed(64))
    y1, l1 = oracle.sfa(q, k, k, idx, 0.125, causal=True)
    y2, l2 = oracle.sfa(q, k, k, idx[..., perm].contiguous(), 0.125, causal=True)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-15)


def test_sfa_weights_sum_to_one():
    """v == 1 everywhere: y == 1 on every row with a surviving slot (softmax weights sum to 1)."""
    B, S1, S2, N1, N2, Dk, Dv, topK = 2, 6, 8, 4, 2, 32, 64, 5
    q, k = _rand((B, S1, N1, Dk), 71), _rand((B, S2, N2, Dk), 72)
    v = torch.ones((B, S2, N2, Dv), dtype=torch.float16)
    g = torch.Generator().manual_seed(73)
    idx = torch.randint(0, S2, (B, S1, N2, topK), generator=g, dtype=torch.int32)
    y, lse = oracle.sfa(q, k, v, idx, 2.0, causal=True)
    alive = np.isfinite(lse)
    np.testing.assert_allclose(y[alive], 1.0, rtol=0, atol=4e-15)
    assert np.all(y[~alive] == 0.0)


def test_sfa_single_survivor_is_exact():
    """topK = 1, or a single unmasked slot: y is exactly that value row, lse is its scaled logit."""
    B, S1, S2, N1, N2, D = 1, 2, 16, 4, 1, 64
    q, k, v = _rand((B, S1, N1, D), 81), _rand((B, S2, N2, D), 82), _rand((B, S2, N2, D), 83)
    idx = torch.tensor([[[[7]], [[2]]]], dtype=torch.int32)  # [1, 2, 1, 1]
    y, lse = oracle.sfa(q, k, v, idx, 0.5)
    y = y.reshape(B, S1, N1, D)
    for s1, j in [(0, 7), (1, 2)]:
        for n1 in range(N1):
            assert np.array_equal(y[0, s1, n1], v[0, j, 0].double().numpy())
            expect = float(torch.dot(q[0, s1, n1].double(), k[0, j, 0].double())) * 0.5
            assert abs(lse[s1 * N1 + n1] - expect) <= 1e-12 * max(1.0, abs(expect))
    # causal: row 0 of (S1=2, S2=16) keeps idx <= 14; only slot 3 survives
    idx2 = torch.tensor([[[[15, 15, 15, 9]], [[15, 3, 3, 3]]]], dtype=torch.int32)
    y2, _ = oracle.sfa(q, k, v, idx2, 0.5, causal=True)
    y2 = y2.reshape(B, S1, N1, D)
    assert np.array_equal(y2[0, 0, 1], v[0, 9, 0].double().numpy())


def test_sfa_zero_query_is_mean_of_values():
    B, S1, S2, N1, N2, Dk, Dv, topK = 1, 4, 10, 2, 1, 32, 32, 6
    q = torch.zeros((B, S1, N1, Dk), dtype=torch.float16)
    k, v = _rand((B, S2, N2, Dk), 91), _rand((B, S2, N2, Dv), 92)
    idx = synth.sample_without_replacement(B * S1 * N2, S2, topK, torch.Generator().manual_seed(93)).view(B, S1, N2, topK)
    y, lse = oracle.sfa(q, k, v, idx, 1.0, causal=True)
    y = y.reshape(B, S1, N1, Dv)
    for s1 in range(S1):
        keep = [int(j) for j in idx[0, s1, 0] if int(j) <= s1 + S2 - S1]
        expect = v[0, keep, 0].double().mean(dim=0).numpy()
        for n1 in range(N1):
            np.testing.assert_allclose(y[0, s1, n1], expect, rtol=1e-14, atol=1e-15)
            assert abs(lse[s1 * N1 + n1] - math.log(len(keep))) < 1e-14


def test_sfa_all_masked_row_outputs_zero():
    B, S1, S2, N1, N2, D = 1, 3, 5, 2, 1, 64
    q, k = _rand((B, S1, N1, D), 101), _rand((B, S2, N2, D), 102)
    # row s1 keeps idx <= s1 + 2; row 0 gets only {3, 4}: every slot masked
    idx = torch.tensor([[[[3, 4, 4]], [[0, 1, 4]], [[4, 4, 4]]]], dtype=torch.int32)
    y, lse = oracle.sfa(q, k, k, idx, 0.1, causal=True)
    y = y.reshape(S1, N1, D)
    assert np.all(y[0] == 0.0) and not np.any(np.signbit(y[0]))
    assert np.all(np.isneginf(lse[:N1]))
    assert np.all(np.isfinite(lse[N1:]))


def test_causal_boundary_slot():
    """The slot at s1 + (S2 - S1) is kept, the one just past it is masked (bottom-right diagonal)."""
    B, S1, S2, N1, N2, D = 1, 3, 8, 1, 1, 64
    q, k, v = _rand((B, S1, N1, D), 111), _rand((B, S2, N2, D), 112), _rand((B, S2, N2, D), 113)
    for s1 in range(S1):
        limit = s1 + S2 - S1
        cand = [limit] + ([limit + 1] if limit + 1 < S2 else [])
        idx = torch.full((B, S1, N2, len(cand)), limit, dtype=torch.int32)
        idx[0, s1, 0] = torch.tensor(cand, dtype=torch.int32)
        y, _ = oracle.sfa(q, k, v, idx, 0.7, causal=True, rows=[s1])
        assert np.array_equal(y[0], v[0, limit, 0].double().numpy())


def test_layouts_agree_bitwise():
    s = synth.SfaShape(B=2, S1=3, S2=40, N1=8, N2=2, Dk=64, Dv=64, topK=12, dtype="bf16", causal=True)
    inp = synth.sfa_inputs(s, seed=3)
    y1, l1 = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], s.scale_value, "BSND", True)
    p = lambda t: t.permute(0, 2, 1, 3).contiguous()
    y2, l2 = oracle.sfa(p(inp["q"]), p(inp["k"]), p(inp["v"]), p(inp["idx"]), s.scale_value, "BNSD", True)
    # BNSD rows come in (b, n1, s1) storage order but the oracle numbers rows (b, s1, n1) for both
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)


def test_value_prefix_view_equals_copy():
    s = synth.SfaShape(B=1, S1=2, S2=64, N1=16, N2=1, Dk=576, Dv=512, topK=20, dtype="bf16",
                       layout="BNSD", causal=True)
    inp = synth.sfa_inputs(s, seed=4)
    assert inp["v"].data_ptr() == inp["k"].data_ptr()  # a view of key
    y1, l1 = oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], s.scale_value, "BNSD", True)
    y2, l2 = oracle.sfa(inp["q"], inp["k"], inp["v"].clone(), inp["idx"], s.scale_value, "BNSD", True)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)


def test_lse_split_merge_identity():
    """Attention over a slot list equals the LSE-weighted merge of attention over any split of it."""
    B, S1, S2, N1, N2, D, topK = 1, 2, 64, 4, 2, 64, 24
    q, k, v = _rand((B, S1, N1, D), 121), _rand((B, S2, N2, D), 122), _rand((B, S2, N2, D), 123)
    idx = synth.sample_without_replacement(B * S1 * N2, S2, topK, torch.Generator().manual_seed(124)).view(B, S1, N2, topK)
    y, lse = oracle.sfa(q, k, v, idx, 0.2)
    parts = [oracle.sfa(q, k, v, idx[..., a:b].contiguous(), 0.2) for a, b in [(0, 7), (7, 8), (8, 24)]]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    Y = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(L, lse, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Y, y, rtol=1e-12, atol=1e-14)


def test_synth_is_seeded_and_without_replacement():
    s = synth.WORKLOADS["tiny"]
    a, b = synth.sfa_inputs(s, seed=0), synth.sfa_inputs(s, seed=0)
    for key in ("q", "k", "idx"):
        assert torch.equal(a[key], b[key])
    assert a["v"] is a["k"]
    rows = a["idx"].reshape(-1, s.topK)
    assert all(len(set(r.tolist())) == s.topK for r in rows)
    assert int(rows.min()) >= 0 and int(rows.max()) < s.S2
    c = synth.sfa_inputs(s, seed=1)
    assert not torch.equal(a["q"], c["q"])


# --- FP8 inputs (BlockSparseAttentionWrapper / VariableBlockSparseAttentionWrapper run:
#     scale_q, scale_k, scale_v per head) --------------------------------------------------

_FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_matches_torch_on_every_code(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes, fmt)
    lib = torch.from_numpy(codes).view(_FP8_TORCH[fmt]).to(torch.float64).numpy()
    assert np.array_equal(ours, lib, equal_nan=True)
    num = ~np.isnan(lib)
    assert np.array_equal(np.signbit(ours[num]), np.signbit(lib[num]))  # -0.0 stays negative


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_specification_values(fmt):
    with open(golden_path("fp8_code_values.json")) as f:
        table = json.load(f)[fmt]
    codes = np.array([int(c, 16) for c, _ in table], dtype=np.uint8)
    want = np.array([float(v) for _, v in table])
    got = oracle.fp8_decode(codes, fmt)
    assert np.array_equal(got, want, equal_nan=True)
    num = ~np.isnan(want)
    assert np.array_equal(np.signbit(got[num]), np.signbit(want[num]))


def _fp8_codes(shape, seed, fmt, spread=1.0):
    """Random FP8 tensor (torch float8 dtype) of N(0, spread^2) values rounded by torch."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * spread).to(_FP8_TORCH[fmt])


@pytest.mark.parametrize("q_fmt,kv_fmt", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_bsr_fp8_matches_sdpa_on_scaled_tensors(q_fmt, kv_fmt):
    # Per-head factors applied by torch to torch's own float8 -> float64 conversion, then
    # SDPA under the BSR mask: an independent statement of the dequantised problem.
    M, N, R, C, Hq, Hkv, D = 12, 16, 4, 4, 4, 2, 64
    indptr = torch.tensor([0, 2, 3, 5], dtype=torch.int32)
    indices = torch.tensor([0, 2, 1, 1, 3], dtype=torch.int32)
    q8 = _fp8_codes((M, Hq, D), 1, q_fmt, 2.0)
    k8 = _fp8_codes((N, Hkv, D), 2, kv_fmt, 2.0)
    v8 = _fp8_codes((N, Hkv, D), 3, kv_fmt)
    sq = torch.tensor([0.5, 0.3, 1.7, 0.11])
    sk = torch.tensor([0.25, 0.9])
    sv = torch.tensor([3.0, 0.07])
    y, lse = oracle.bsr_fp8(q8, k8, v8, q_fmt, kv_fmt, sq, sk, sv, indptr, indices, R, C)
    qd = q8.to(torch.float64) * sq.double()[None, :, None]
    kd = k8.to(torch.float64) * sk.double()[None, :, None]
    vd = v8.to(torch.float64) * sv.double()[None, :, None]
    mask = torch.from_numpy(oracle.bsr_mask(indptr, indices, M, N, R, C))
    bias = _bias_from_bool(mask)[None]
    ref = _sdpa(qd.permute(1, 0, 2), kd.permute(1, 0, 2), vd.permute(1, 0, 2), bias, 1 / 8)  # [Hq, M, D]
    np.testing.assert_allclose(y.reshape(M, Hq, D), ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
    assert np.isfinite(lse).all()


def test_bsr_fp8_uniform_scales_fold_into_logit_scale_and_output():
    # softmax(a q . b k * s) (c v) = c * attention with logit scale s a b: closed form of the
    # three factors, against the unscaled oracle on the decoded values.
    M, N, R, C, Hq, Hkv, D = 8, 8, 4, 4, 2, 1, 64
    indptr = torch.tensor([0, 1, 3], dtype=torch.int32)
    indices = torch.tensor([0, 0, 1], dtype=torch.int32)
    q8 = _fp8_codes((M, Hq, D), 4, "e4m3")
    k8 = _fp8_codes((N, Hkv, D), 5, "e4m3")
    v8 = _fp8_codes((N, Hkv, D), 6, "e4m3")
    a, b, c = 0.75, 1.25, 4.0
    y, lse = oracle.bsr_fp8(q8, k8, v8, "e4m3", "e4m3", torch.full((Hq,), a), torch.full((Hkv,), b),
                            torch.full((Hkv,), c), indptr, indices, R, C, sm_scale=0.1)
    y1, lse1 = oracle.bsr(oracle.fp8_dequant(q8, "e4m3"), oracle.fp8_dequant(k8, "e4m3"),
                          oracle.fp8_dequant(v8, "e4m3"), indptr, indices, R, C, sm_scale=0.1 * a * b)
    np.testing.assert_allclose(y, c * y1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse1, rtol=1e-12)


def test_vbsr_fp8_heads_first_layout_matches_sdpa():
    Hq, Hkv, D = 4, 2, 64
    bmap = torch.tensor([[[1, 0], [1, 1]], [[0, 1], [1, 0]]], dtype=torch.bool)
    rs = torch.tensor([[3, 5], [6, 2]], dtype=torch.int32)
    cs = torch.tensor([[4, 4], [2, 6]], dtype=torch.int32)
    M, N = 8, 8
    q8 = _fp8_codes((Hq, M, D), 7, "e4m3")
    k8 = _fp8_codes((Hkv, N, D), 8, "e5m2")
    v8 = _fp8_codes((Hkv, N, D), 9, "e5m2")
    sq, sk, sv = torch.tensor([1.0, 0.5, 2.0, 0.25]), torch.tensor([0.3, 1.1]), torch.tensor([2.0, 0.6])
    y, _ = oracle.vbsr_fp8(q8, k8, v8, "e4m3", "e5m2", sq, sk, sv, bmap, rs, cs)
    qd = q8.to(torch.float64) * sq.double()[:, None, None]
    kd = k8.to(torch.float64) * sk.double()[:, None, None]
    vd = v8.to(torch.float64) * sv.double()[:, None, None]
    mask = torch.from_numpy(oracle.variable_block_mask(bmap, rs, cs))  # [Hkv, M, N]
    bias = _bias_from_bool(mask.repeat_interleave(Hq // Hkv, dim=0))
    ref = _sdpa(qd, kd, vd, bias, 1 / 8)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_index_report_on_a_constructed_tensor():
    # BSND [B=1, S1=2, N2=2, topK=4], S2 = 10: row (0,0,0) clean, (0,0,1) one index repeated,
    # (0,1,0) two slots out of range (-1 and 10), (0,1,1) out of range and a repeat
    idx = torch.tensor([[[[0, 3, 9, 5], [2, 2, 7, 1]],
                         [[-1, 4, 10, 6], [8, 8, 11, 0]]]], dtype=torch.int32)
    assert oracle.index_report(idx, 10) == {"out_of_range": 3, "duplicate_rows": 2}
    # the same rows in BNSD order give the same report
    assert oracle.index_report(idx.permute(0, 2, 1, 3), 10, "BNSD") == {"out_of_range": 3, "duplicate_rows": 2}
    # the workload recipe draws without replacement inside the range
    inp = synth.sfa_inputs(synth.WORKLOADS["tiny"], seed=0)
    assert oracle.index_report(inp["idx"], 64) == {"out_of_range": 0, "duplicate_rows": 0}
