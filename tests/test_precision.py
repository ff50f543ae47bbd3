"""The precision standard (SparseFlashAttention page, section 4) as implemented by oracle.precision."""
import json

import numpy as np
import torch

from oracle import precision
from tests.conftest import golden_path


def test_thresholds_match_page_table():
    ex = json.load(open(golden_path("precision_standard.json")))
    for name, text in ex["thresholds"].items():
        base, exp = text.split("^")
        assert precision.THRESHOLDS[name] == float(base) ** float(exp)
    assert precision.GUARD == ex["guard"]


def test_literal_metrics_hand_example():
    golden = np.array([1.0, -2.0, 0.0, 4.0])
    actual = np.array([1.001, -2.0, 1e-7, 3.0])
    e = [0.001 / (1.0 + 1e-7), 0.0, 1e-7 / 1e-7, 1.0 / (4.0 + 1e-7)]
    mere, mare = precision.mere_mare(actual, golden)
    assert abs(mere - sum(e) / 4) < 1e-15
    assert abs(mare - 1.0) < 1e-15


def test_gate_accepts_exact_rounding_and_rejects_planted_errors():
    g = torch.Generator().manual_seed(0)
    golden = (torch.randn(200_000, generator=g, dtype=torch.float64) * 0.05).numpy()
    for dt, tdt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
        rounded = torch.from_numpy(golden).to(tdt).double().numpy()
        rep = precision.gate(rounded, golden, dt)
        assert rep["pass"], rep
        thr = precision.THRESHOLDS[dt]
        # a uniform relative error of 2*Thr breaks MERE
        assert not precision.gate(golden * (1 + 2 * thr), golden, dt)["pass"]
        # an absolute error of RMS * Thr on every element breaks the tau rule near zero
        bad = golden + np.sqrt(np.mean(golden ** 2)) * thr
        assert not precision.gate(bad, golden, dt)["pass"]
    # non-finite output fails
    x = golden.copy()
    x[3] = np.nan
    assert not precision.gate(x, golden, "fp16")["pass"]
