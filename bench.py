#!/usr/bin/env python3
"""Throughput of the sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

A step is one sparse-attention call (index read, causal mask, gather, QK^T,
online softmax, PV, split-K merge, output) over one batch of the workload, with
all inputs already resident in HBM.  The default workload is the GQA decode
problem (B=32, S1=1, S2=8192, N1=32, N2=8, D=128, topK=1024, bf16, BSND).  To
keep the gathered rows from being served by the 256 MB Infinity Cache, steps
rotate over several independent input sets whose distinct gathered bytes
exceed twice the cache.

Prints one JSON line: the gathered-KV bandwidth (GB/s) as ``value``, the
kernel's roofline figures (HIP events on the launch stream), and the fp64 CPU
oracle timed on a bounded sample on this host (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_13_amd import api, binding, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0}
MALL_BYTES = 256 << 20


KERNEL_SOURCES = ("sparse_attention_13_amd/csrc/common.hpp", "sparse_attention_13_amd/csrc/topk_kernel.hpp",
                  "sparse_attention_13_amd/csrc/topk_dvs.hpp", "sparse_attention_13_amd/csrc/topk_launch.hpp",
                  "sparse_attention_13_amd/csrc/api.hip", "sparse_attention_13_amd/build.py")


def kernel_source_sha256() -> str:
    """Hash of the sources that define the top-K kernels, their launch configuration and their
    compile flags."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is none or the kernel
    sources changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"topk_fwd_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_h = re.search(r"^source_sha256: ([0-9a-f]{64})$", text, re.M)
    if not m_t or not m_h or m_h.group(1) != kernel_source_sha256():
        return None
    return int(m_t.group(1))


def topk_work(shape: synth.SfaShape, idx: torch.Tensor) -> dict:
    """Algorithmic work of one call: unmasked slots only; V rows counted only when V is not
    a view of K (then one gathered row serves both)."""
    s = shape
    if s.layout == "BNSD":
        idx = idx.permute(0, 2, 1, 3)
    idx = idx.to("cpu")
    if s.causal:
        limit = torch.arange(s.S1).view(1, s.S1, 1, 1) + (s.S2 - s.S1)
        valid = (idx <= limit).sum().item()
    else:
        valid = idx.numel()
    row_bytes = s.Dk * 2 + (0 if s.value == "alias" else s.Dv * 2)
    gathered = valid * row_bytes
    idx_bytes = idx.numel() * 4
    qo_bytes = s.B * s.S1 * s.N1 * (s.Dk + s.Dv) * 2
    flops = valid * s.G * 2 * (s.Dk + s.Dv)
    return {"valid_slots": int(valid), "gathered_bytes": int(gathered), "alg_bytes": int(gathered + idx_bytes + qo_bytes),
            "flops": int(flops)}


def identity_indices(shape: synth.SfaShape) -> torch.Tensor:
    """Every key of the sequence in order (topK = S2): the dense operator through the sparse path."""
    s = shape
    ar = torch.arange(s.S2, dtype=torch.int32)
    if s.layout == "BSND":
        return ar.view(1, 1, 1, s.S2).expand(s.B, s.S1, s.N2, s.S2).contiguous()
    return ar.view(1, 1, 1, s.S2).expand(s.B, s.N2, s.S1, s.S2).contiguous()


class TopkSets:
    """R independent device-resident input sets of one workload, plus outputs and workspace.
    identity: the shape's topK is S2 and the indices select every key in order."""

    def __init__(self, shape: synth.SfaShape, n_sets: int, dev: str, identity: bool = False):
        self.shape = shape
        self.sets = []
        for r in range(n_sets):
            if identity:
                inp = synth.sfa_inputs(dataclasses.replace(shape, topK=1), seed=100 + r)
                inp["idx"] = identity_indices(shape)
            else:
                inp = synth.sfa_inputs(shape, seed=100 + r)
            progress(f"  input set {r + 1}/{n_sets}")
            k = inp["k"].to(dev)
            if inp["v"] is inp["k"]:
                v = k
            elif inp["v"].data_ptr() == inp["k"].data_ptr():
                v = k[..., : shape.Dv]
            else:
                v = inp["v"].to(dev)
            self.sets.append({"q": inp["q"].to(dev), "k": k, "v": v, "idx": inp["idx"].to(dev), "cpu": inp})
        s0 = self.sets[0]
        self.out = [api.sparse_flash_attention(st["q"], st["k"], st["v"], st["idx"], shape.scale_value,
                                               shape.layout, shape.causal) for st in self.sets[:1]][0]
        self.lse = None
        need = api.workspace_bytes(s0["q"], s0["k"], s0["v"], s0["idx"], shape.layout, shape.causal)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

        s = shape
        self.calls = [api.sparse_flash_attention(st["q"], st["k"], st["v"], st["idx"], s.scale_value, s.layout,
                                                 s.causal, out=self.out, workspace=self.ws, prepare=True)
                      for st in self.sets]
        self.stream = torch.cuda.current_stream().cuda_stream

    def step(self, i: int):
        self.calls[i % len(self.calls)](self.stream)


def n_rotation_sets(shape: synth.SfaShape, work: dict) -> int:
    k_bytes = shape.B * shape.S2 * shape.N2 * shape.Dk * 2
    distinct = min(k_bytes, work["gathered_bytes"])
    # distinct gathered bytes across the rotation must exceed 2x the Infinity Cache
    return int(min(8, max(2, math.ceil(2 * MALL_BYTES / max(distinct, 1)))))


def time_steps(step, n_steps: int, n_warmup: int):
    """Runs n_warmup untimed steps, then times n_steps back to back: wall clock between two
    synchronisations, and the GPU timeline between two HIP events recorded on the launch
    stream at the ends of the timed region (per-step events would add their own gaps).
    Returns (wall ms per step, GPU ms per step)."""
    for i in range(n_warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(n_steps):
        step(n_warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / n_steps, start.elapsed_time(end) / n_steps


def cpu_baseline_topk(shape: synth.SfaShape, sets: TopkSets, work: dict, budget_s: float = 12.0) -> dict:
    import oracle

    inp = sets.sets[0]["cpu"]
    nrows = shape.B * shape.S1 * shape.N1
    threads = oracle.default_threads()
    # calibrate on a small slice, then size the sample to the time budget
    probe = np.arange(0, nrows, max(1, nrows // 64))[:64]
    t0 = time.perf_counter()
    oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], shape.scale_value, shape.layout, shape.causal,
               rows=probe, nthreads=threads)
    dt_probe = max(time.perf_counter() - t0, 1e-4)
    want = len(probe) * budget_s / dt_probe
    n = int(min(nrows, max(len(probe), want)))
    rows = np.linspace(0, nrows - 1, n).astype(np.int64)
    # a workload the oracle finishes quickly runs whole, repeated until the budget is spent
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], shape.scale_value, shape.layout, shape.causal,
                   rows=rows, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 0.8 * budget_s or reps >= 200:
            break
    frac = n * reps / nrows
    return {"value": work["gathered_bytes"] * frac / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {nrows} query rows of the same inputs, {reps} pass(es) (fp64 scalar C, {threads} "
                      f"threads), {dt:.1f} s; rate = gathered-KV bytes of the sampled rows / time",
            "tflops": work["flops"] * frac / dt / 1e12}


def progress(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bench_topk(name: str, steps: int, warmup: int, with_cpu: bool, dev: str, dense: bool = False) -> dict:
    """dense: the same workload with topK = S2 and identity indices (dense attention through the
    same kernels, the comparison baseline of the sparse form); its keys are L2/MALL-resident,
    so two input sets rotate."""
    shape = synth.WORKLOADS[name]
    if dense:
        shape = dataclasses.replace(shape, topK=shape.S2, sorted_indices=True)
        name = name + "_dense"
    progress(f"{name}: generating inputs")
    if dense:
        work = topk_work(shape, identity_indices(shape))
        n_sets = 2
    else:
        probe = synth.sfa_inputs(shape, seed=100)
        work = topk_work(shape, probe["idx"])
        del probe
        n_sets = n_rotation_sets(shape, work)
    sets = TopkSets(shape, n_sets, dev, identity=dense)
    progress(f"{name}: {len(sets.sets)} input sets resident, timing {steps} steps")
    ms_step, ms_kernel_mean = time_steps(sets.step, steps, warmup)
    gbs = work["gathered_bytes"] / (ms_step * 1e-3) / 1e9
    tflops = work["flops"] / (ms_step * 1e-3) / 1e12
    alg_gbs_kernel = work["alg_bytes"] / (ms_kernel_mean * 1e-3) / 1e9
    res = {
        "workload": name,
        "ms_per_step": ms_step,
        "ms_kernel_mean": ms_kernel_mean,
        "gathered_GBs": gbs,
        "gathered_frac_hbm": gbs / HBM_PEAK_GBS,
        "TFLOPs": tflops,
        "frac_mfma": tflops / MFMA_PEAK_TFLOPS[shape.dtype],
        "alg_bytes": work["alg_bytes"],
        "gathered_bytes": work["gathered_bytes"],
        "flops": work["flops"],
        "rotation_sets": len(sets.sets),
        "roofline": {"bound": "hbm", "achieved": alg_gbs_kernel, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg_gbs_kernel / HBM_PEAK_GBS, "traffic": measured_traffic(name)},
    }
    progress(f"{name}: {ms_step * 1e3:.1f} us/step, {gbs:.0f} GB/s gathered, {tflops:.1f} TFLOP/s")
    if with_cpu:
        progress(f"{name}: timing the fp64 CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_topk(shape, sets, work)
    del sets
    torch.cuda.empty_cache()
    return res


def bsr_work(shape: synth.BsrShape, indptr: torch.Tensor, mask: torch.Tensor = None) -> dict:
    """Algorithmic work of one BSR call: every allowed (query, key) pair of every query head,
    QK^T and PV; block loads of K and V per (block row, kv head).  mask: optional per-block
    mask [nnz, R, C]; its clear elements are not counted."""
    s = shape
    ip = indptr.tolist()
    MB = len(ip) - 1
    pairs = 0
    for br in range(MB):
        rows = min(s.R, s.M - br * s.R)
        if mask is None:
            pairs += rows * (ip[br + 1] - ip[br]) * s.C
        else:
            pairs += int(mask[ip[br]:ip[br + 1], :rows].sum())
    flops = pairs * s.Hq * 4 * s.D
    block_bytes = ip[-1] * s.C * s.Hkv * s.D * 2 * 2
    qo_bytes = s.M * s.Hq * s.D * 2 * 2
    return {"flops": int(flops), "alg_bytes": int(block_bytes + qo_bytes), "pairs": int(pairs)}


def bench_bsr(name: str, steps: int, warmup: int, dev: str, mask_density: float = 0.0, fp8: str = "") -> dict:
    """mask_density > 0: a per-block mask whose elements are set with that probability.
    fp8 ("e4m3" / "e5m2"): FP8 q, k, v with per-head factors (the expansion to fp16 copies is
    part of every timed step)."""
    shape = synth.WORKLOADS[name]
    progress(f"{name}{' fp8 ' + fp8 if fp8 else ''}: generating inputs")
    sets = []
    for r in range(2):
        inp = synth.bsr_fp8_inputs(shape, fp8, fp8, seed=200 + r) if fp8 else synth.bsr_inputs(shape, seed=200 + r)
        if mask_density > 0:
            g = torch.Generator().manual_seed(300 + r)
            inp["mask"] = torch.rand((len(inp["indices"]), shape.R, shape.C), generator=g) < mask_density
        sets.append({k: (v.to(dev) if k in ("q", "k", "v", "scale_q", "scale_k", "scale_v") else v)
                     for k, v in inp.items()})
    work = bsr_work(shape, sets[0]["indptr"], sets[0].get("mask"))
    wrappers = []
    for st in sets:
        w = api.BlockSparseAttentionWrapper()
        w.plan(st["indptr"], st["indices"], shape.M, shape.N, shape.R, shape.C, shape.Hq, shape.Hkv, shape.D,
               mask=st.get("mask"), causal=shape.causal,
               q_data_type=st["q"].dtype if fp8 else synth.DTYPES[shape.dtype])
        wrappers.append(w)
    out = torch.empty(tuple(sets[0]["q"].shape), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    def step(i):
        st = sets[i % len(sets)]
        if fp8:
            wrappers[i % len(sets)].run(st["q"], st["k"], st["v"], scale_q=st["scale_q"], scale_k=st["scale_k"],
                                        scale_v=st["scale_v"], out=out)
        else:
            wrappers[i % len(sets)].run(st["q"], st["k"], st["v"], out=out)

    progress(f"{name}: timing {steps} steps")
    ms_step, ms_kernel_mean = time_steps(step, steps, warmup)
    tflops = work["flops"] / (ms_step * 1e-3) / 1e12
    tflops_k = work["flops"] / (ms_kernel_mean * 1e-3) / 1e12
    progress(f"{name}: {ms_step * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s")
    res = {"ms_per_step": ms_step, "ms_kernel_mean": ms_kernel_mean, "TFLOPs": tflops,
           "frac_mfma": tflops_k / MFMA_PEAK_TFLOPS[shape.dtype], "flops": work["flops"],
           "alg_bytes": work["alg_bytes"],
           "roofline": {"bound": "mfma", "achieved": tflops_k, "peak": MFMA_PEAK_TFLOPS[shape.dtype],
                        "unit": "TFLOP/s", "frac": tflops_k / MFMA_PEAK_TFLOPS[shape.dtype],
                        "traffic": measured_traffic("bsr") if not fp8 and mask_density == 0 else None}}
    if fp8:
        # FP8 inputs: q, k, v read once as 1-byte codes; the compute runs on fp16 MFMA
        res["input_dtype"] = "fp8_" + fp8
        res["fp8_input_bytes"] = int(sum(sets[0][k].numel() for k in ("q", "k", "v")))
    return res


def vbsr_work(shape: synth.VbsrShape, inp: dict) -> dict:
    """Algorithmic work of one variable block-sparse call: every allowed (query, key) pair of
    every query head (causal pairs excluded), QK^T and PV; K and V rows loaded once per (block
    row, KV head)."""
    s = shape
    G = s.Hq // s.Hkv
    bm, rs, cs = inp["block_mask_map"], inp["block_row_sz"].long(), inp["block_col_sz"].long()
    pairs, loads = 0, 0
    for h in range(s.Hkv):
        keys = (bm[h].long() * cs[h][None, :]).sum(dim=1)  # keys per block row
        pairs += int((rs[h] * keys).sum())
        loads += int(keys[rs[h] > 0].sum())
    if s.causal:
        raise ValueError("the causal variable-block work count is not implemented")
    flops = pairs * G * 4 * s.D
    kv_bytes = loads * s.D * 2 * (1 if s.value == "alias" else 2)
    qo_bytes = s.M * s.Hq * s.D * 2 * 2
    return {"flops": int(flops), "alg_bytes": int(kv_bytes + qo_bytes), "pairs": int(pairs)}


def bench_vbsr(steps: int, warmup: int, dev: str) -> dict:
    shape = synth.VBSR_WORKLOAD
    progress("vbsr: generating inputs")
    sets, wrappers = [], []
    for r in range(2):
        inp = synth.vbsr_inputs(shape, seed=400 + r)
        w = api.VariableBlockSparseAttentionWrapper()
        w.plan(inp["block_mask_map"], inp["block_row_sz"], inp["block_col_sz"], shape.Hq, shape.Hkv, shape.D,
               causal=shape.causal, q_data_type=synth.DTYPES[shape.dtype])
        wrappers.append(w)
        sets.append(inp)
    work = vbsr_work(shape, sets[0])
    dsets = [{k: inp[k].to(dev) for k in ("q", "k", "v")} for inp in sets]
    out = torch.empty_like(dsets[0]["q"])
    torch.cuda.synchronize()

    def step(i):
        st = dsets[i % 2]
        wrappers[i % 2].run(st["q"], st["k"], st["v"], out=out)

    progress(f"vbsr: timing {steps} steps")
    ms_step, ms_kernel_mean = time_steps(step, steps, warmup)
    tflops = work["flops"] / (ms_step * 1e-3) / 1e12
    tflops_k = work["flops"] / (ms_kernel_mean * 1e-3) / 1e12
    progress(f"vbsr: {ms_step * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s")
    return {"ms_per_step": ms_step, "ms_kernel_mean": ms_kernel_mean, "TFLOPs": tflops,
            "frac_mfma": tflops_k / MFMA_PEAK_TFLOPS[shape.dtype], "flops": work["flops"],
            "alg_bytes": work["alg_bytes"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_decode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="also time the other top-K workloads (extra key)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)
        return
    binding.load()
    if args.workload == "bsr":
        # the block-sparse workload alone: MFMA-bound, reported in TFLOP/s (no CPU leg)
        res = bench_bsr("bsr", args.steps, args.warmup, dev)
        shape = synth.WORKLOADS["bsr"]
        achieved = res["flops"] / (res["ms_kernel_mean"] * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[shape.dtype]
        print(json.dumps({
            "metric": "sparse-attn TFLOP/s + gathered-KV HBM GB/s (% of MI355X peak), per config",
            "value": round(res["TFLOPs"], 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": shape.dtype,
            "data": "synthetic (seeded N(0,1) q/k/v, diagonal + uniform column blocks per block row)",
            "config": {"workload": "bsr", "M": shape.M, "N": shape.N, "R": shape.R, "C": shape.C, "Hq": shape.Hq,
                       "Hkv": shape.Hkv, "D": shape.D, "blocks_per_row": shape.blocks_per_row,
                       "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                         "frac": achieved / peak, "traffic": measured_traffic("bsr")},
            "cpu_baseline": None}), flush=True)
        return
    main_res = bench_topk(args.workload, args.steps, args.warmup, not args.no_cpu_baseline, dev)
    shape = synth.WORKLOADS[args.workload]
    line = {
        "metric": "sparse-attn TFLOP/s + gathered-KV HBM GB/s (% of MI355X peak), per config",
        "value": round(main_res["gathered_GBs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded N(0,1) q/k, uniform top-K indices without replacement)",
        "config": {"workload": args.workload, "B": shape.B, "S1": shape.S1, "S2": shape.S2, "N1": shape.N1,
                   "N2": shape.N2, "Dk": shape.Dk, "Dv": shape.Dv, "topK": shape.topK, "layout": shape.layout,
                   "causal": shape.causal, "parallelism": "single GPU"},
        "tflops": round(main_res["TFLOPs"], 3),
        "frac_hbm_gathered": round(main_res["gathered_frac_hbm"], 4),
        "roofline": main_res["roofline"],
        "cpu_baseline": main_res.get("cpu_baseline"),
    }
    if args.all:
        extra = {}
        for name in ("tiny", "gqa_decode", "mla_decode", "gqa_prefill"):
            if name == args.workload:
                continue
            r = bench_topk(name, args.steps, args.warmup, False, dev)
            extra[name] = {k: r[k] for k in ("ms_per_step", "ms_kernel_mean", "gathered_GBs", "gathered_frac_hbm",
                                             "TFLOPs", "frac_mfma", "rotation_sets", "roofline")}
            if name == "gqa_prefill":
                # its gathered rows come from L2/MALL (HBM traffic is 0.05 of them), so HBM does not
                # bound it: report it against the MFMA roofline, as the target does
                achieved = r["flops"] / (r["ms_kernel_mean"] * 1e-3) / 1e12
                peak = MFMA_PEAK_TFLOPS[synth.WORKLOADS[name].dtype]
                extra[name]["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                                           "frac": achieved / peak, "traffic": r["roofline"]["traffic"]}
        # the pages' claim O(S1 S2 D) -> O(S1 topK D): the prefill shape with every key selected
        r = bench_topk("gqa_prefill", args.steps, args.warmup, False, dev, dense=True)
        extra["gqa_prefill_dense"] = {k: r[k] for k in ("ms_per_step", "ms_kernel_mean", "TFLOPs", "frac_mfma")}
        if "gqa_prefill" in extra:
            extra["gqa_prefill_dense"]["sparse_speedup"] = r["ms_per_step"] / extra["gqa_prefill"]["ms_per_step"]
        extra["bsr"] = bench_bsr("bsr", args.steps, args.warmup, dev)
        extra["bsr_masked_0.5"] = bench_bsr("bsr", args.steps, args.warmup, dev, mask_density=0.5)
        extra["bsr_fp8_e4m3"] = bench_bsr("bsr", args.steps, args.warmup, dev, fp8="e4m3")
        extra["vbsr"] = bench_vbsr(args.steps, args.warmup, dev)
        line["per_config"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
