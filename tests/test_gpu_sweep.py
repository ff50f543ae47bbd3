"""Seeded random sweep over the supported problem space (head-dim pairs, GQA group sizes,
layouts, dtypes, causal, aliased or separate values, ragged topK and block-sparse patterns
with and without per-block masks), each case against the fp64 oracle under the precision
gate.  The draws reach the kernels' head tilings, ring depths, split counts and the
wide-value kernel."""
import random

import numpy as np
import pytest
import torch

from sparse_attention_13_amd import synth
from tests.test_gpu_bsr import run_bsr
from tests.test_gpu_topk import log, run_and_compare

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (192, 128), (192, 192), (256, 256), (512, 512), (576, 512)]


def _topk_case(seed):
    rng = random.Random(seed)
    Dk, Dv = rng.choice(DIMS)
    G = rng.choice([1, 2, 3, 4, 8, 16, 24, 32, 48, 64, 96, 128])
    N2 = rng.choice([1, 2]) if G <= 32 else 1
    B = rng.choice([1, 2, 3])
    S1 = rng.choice([1, 2, 3, 5])
    S2 = rng.randint(max(S1, 40), 1500)
    topK = rng.randint(1, min(S2, 700))
    dtype = rng.choice(["fp16", "bf16"])
    layout = rng.choice(["BSND", "BNSD"])
    causal = rng.random() < 0.5
    value = "alias" if rng.random() < 0.7 else "separate"  # alias: v is k, or the view k[..., :Dv]
    # keep the oracle's work near a second
    while B * S1 * N2 * G * topK * (Dk + Dv) > 3e8 and topK > 1:
        topK = max(1, topK // 2)
    return synth.SfaShape(B=B, S1=S1, S2=S2, N1=G * N2, N2=N2, Dk=Dk, Dv=Dv, topK=topK, dtype=dtype,
                          layout=layout, causal=causal, value=value, sorted_indices=rng.random() < 0.3)


@pytest.mark.parametrize("seed", range(40))
def test_random_topk_shapes(seed):
    shape = _topk_case(1000 + seed)
    log(f"sweep seed {seed}")
    run_and_compare(shape, seed=seed)


# head-dim pairs with no kernel of their own: they run on the smallest compiled pair that covers
# them, with q zero past Dk and output columns past Dv left unwritten
PADDED_DIMS = [(128, 64), (192, 64), (256, 128), (256, 192), (320, 256), (320, 320), (384, 384), (448, 192),
               (448, 448), (512, 256), (576, 576), (576, 64)]


@pytest.mark.parametrize("seed", range(len(PADDED_DIMS)))
def test_padded_head_dims(seed):
    shape = _topk_case(3000 + seed)
    Dk, Dv = PADDED_DIMS[seed]
    rng = random.Random(seed)
    G = rng.choice([1, 4, 8, 16, 32, 64, 128])
    N2 = 1 if G > 16 else rng.choice([1, 2])
    topK = shape.topK
    while shape.B * shape.S1 * N2 * G * topK * (Dk + Dv) > 3e8 and topK > 1:
        topK = max(1, topK // 2)
    shape = synth.SfaShape(B=shape.B, S1=shape.S1, S2=shape.S2, N1=G * N2, N2=N2, Dk=Dk, Dv=Dv, topK=topK,
                           dtype=shape.dtype, layout=shape.layout, causal=shape.causal, value=shape.value,
                           sorted_indices=shape.sorted_indices)
    log(f"padded head dims {Dk}/{Dv}")
    run_and_compare(shape, seed=seed)


@pytest.mark.parametrize("Dk,Dv,G,causal", [(448, 384, 64, True), (320, 256, 128, False)])
def test_padded_head_dims_wide_value_kernel(Dk, Dv, G, causal):
    # many query vectors with wide values: the wide-value kernel (compiled for 512 / 512) with
    # the call's head dims at run time, value the prefix view key[..., :Dv]
    shape = synth.SfaShape(B=2, S1=2, S2=900, N1=G, N2=1, Dk=Dk, Dv=Dv, topK=300, dtype="bf16", layout="BNSD",
                           causal=causal, value="alias", sorted_indices=True)
    log(f"padded head dims {Dk}/{Dv}, G={G} (wide-value kernel)")
    run_and_compare(shape, seed=7)


def _bsr_case(seed):
    rng = random.Random(seed)
    R = rng.choice([1, 4, 8, 16, 32, 64])
    C = rng.choice([1, 8, 16, 32, 64])
    NB = rng.randint(1, 12)
    N = NB * C
    causal = rng.random() < 0.3
    M = rng.randint(1, N if causal else 2 * N)
    Hkv = rng.choice([1, 2])
    Hq = Hkv * rng.choice([1, 2, 4])
    D = rng.choice([64, 128, 256])
    MB = (M + R - 1) // R
    g = torch.Generator().manual_seed(seed)
    indptr, indices = [0], []
    for _ in range(MB):
        k = rng.randint(0, NB)
        indices += sorted(torch.randperm(NB, generator=g)[:k].tolist())
        indptr.append(len(indices))
    mask = None
    if rng.random() < 0.3 and len(indices):
        mask = torch.rand((len(indices), R, C), generator=g) < 0.6
    return M, N, R, C, Hq, Hkv, D, indptr, indices, causal, mask


@pytest.mark.parametrize("seed", range(16))
def test_random_bsr_shapes(seed):
    M, N, R, C, Hq, Hkv, D, indptr, indices, causal, mask = _bsr_case(2000 + seed)
    _bsr_run_case(seed, M, N, R, C, Hq, Hkv, D, indptr, indices, causal, mask)


@pytest.mark.parametrize("seed,D", [(0, 320), (1, 384), (2, 448), (3, 576), (4, 192)])
def test_bsr_padded_head_dims(seed, D):
    M, N, R, C, Hq, Hkv, _, indptr, indices, causal, mask = _bsr_case(2500 + seed)
    if D > 256 and mask is not None and R * Hq // Hkv > 32 and D <= 512:
        mask = None  # masked plans of wide heads with many query vectors per item are not supported
    _bsr_run_case(seed, M, N, R, C, Hq, Hkv, D, indptr, indices, causal, mask)


def _bsr_run_case(seed, M, N, R, C, Hq, Hkv, D, indptr, indices, causal, mask):
    g = torch.Generator().manual_seed(seed)
    dt = torch.float16 if seed % 2 == 0 else torch.bfloat16
    q = torch.randn((M, Hq, D), generator=g).to(dt)
    k = torch.randn((N, Hkv, D), generator=g).to(dt)
    v = torch.randn((N, Hkv, D), generator=g).to(dt)
    run_bsr(q, k, v, indptr, indices, M, N, R, C, causal=causal, dtype="fp16" if seed % 2 == 0 else "bf16",
            tag=f"sweep{seed}", mask=mask)
