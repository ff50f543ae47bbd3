#!/usr/bin/env python3
"""Throughput of the sparse-attention hot path on one MI355X, per workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--no-cpu-baseline] [--with-ceilings | --ceilings] [--copy-calibration BYTES]

A step is one call of the library (index read, causal mask, gather, QK^T, online softmax,
PV, split-K merge, output) over one batch of a workload, with all inputs already resident
in HBM.  The default run times the five workloads: GQA decode (the headline line, B=32 S1=1
S2=8192 N1=32 N2=8 D=128 topK=1024 bf16 BSND) and, under ``per_config``, the tiny problem,
MLA decode, GQA prefill and the BSR block-sparse workload.  Every entry carries:

  * the step time: wall clock over K back-to-back steps, the GPU timeline of the same region
    (two HIP events on the launch stream), and the median / p10 / p90 of K individually
    bracketed steps;
  * ``roofline``: algorithmic bytes (HBM-bound workloads) or flops (MFMA-bound ones) per
    call over the GPU time, against MI355X peak (8 TB/s HBM, 2.5 PFLOP/s dense fp16/bf16),
    and the profiled HBM traffic; with ``--with-ceilings`` also the measured practical
    ceiling of the same kind of work (gather / copy / MFMA microbenchmarks of
    libsfa_ubench.so, run in the same process);
  * ``cpu_baseline``: the fp64 CPU oracle timed on a bounded sample of the same inputs on this
    host's cores (multi-threaded, and single-threaded on a smaller sample), as a rate in the
    entry's unit; the CPU model and core count are reported.

Steps rotate over input sets whose distinct gathered bytes exceed twice the 256 MB Infinity
Cache, so gathered rows of the decode workloads come from HBM.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import glob
import hashlib
import json
import math
import os
import re
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
METRIC = "sparse-attn TFLOP/s + gathered-KV HBM GB/s (% of MI355X peak), per config"
PROFILE_KERNELS = {"gqa_decode": "topk_fwd", "mla_decode": "topk_fwd_dvs", "gqa_prefill": "topk_fwd",
                   "bsr": "topk_fwd", "tiny": "topk_fwd", "vbsr": "topk_fwd", "dense": "topk_fwd"}


def progress(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
# provenance of the profiled traffic figures

def kernel_source_sha256() -> str:
    """Hash of every source that defines the kernels, their launch configuration and their
    compile flags (the library's HIP units and headers, and the build script)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "sparse_attention_13_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "sparse_attention_13_amd", "csrc", "*.hpp")))
    files.append(os.path.join(ROOT, "sparse_attention_13_amd", "build.py"))
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or None when there is none or the kernel sources changed since."""
    kern = PROFILE_KERNELS.get(workload, "topk_fwd")
    path = os.path.join(ROOT, "profiles", f"{kern}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_h = re.search(r"^source_sha256: ([0-9a-f]{64})$", text, re.M)
    if not m_t or not m_h or m_h.group(1) != kernel_source_sha256():
        return None
    return int(m_t.group(1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------------------------
# timing

def time_steps(step, n_steps: int, n_warmup: int) -> dict:
    """n_warmup untimed steps; then n_steps back to back (wall clock between two
    synchronisations and GPU time between two events on the launch stream); then n_steps more,
    each bracketed by its own event pair (for the distribution; the pairs add their own gaps
    between steps, not inside them).  Times in ms per step."""
    for i in range(n_warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(n_steps):
        step(n_warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(n_warmup + n_steps + i)
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    return {"ms_wall": (t1 - t0) * 1e3 / n_steps, "ms_gpu_mean": start.elapsed_time(end) / n_steps,
            "ms_step_median": float(np.median(per)), "ms_step_p10": float(np.percentile(per, 10)),
            "ms_step_p90": float(np.percentile(per, 90))}


# ---------------------------------------------------------------------------------------------
# practical ceilings (microbenchmarks in libsfa_ubench.so)

class Ceilings:
    """Copy, random-row gather and MFMA microbenchmarks; None where the library is missing."""

    def __init__(self):
        path = os.path.join(ROOT, "sparse_attention_13_amd", "libsfa_ubench.so")
        self.lib = None
        if os.path.exists(path):
            lib = ctypes.CDLL(path)
            P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
            lib.ub_copy_run.argtypes = [P, P, L, P]
            lib.ub_gather_run.argtypes = [I, I, P, P, I, I, I, I, I, L, L, I, P, P]
            lib.ub_gather_reg_threads.argtypes = [I]
            lib.ub_mfma_run.argtypes = [I, I, I, P, P]
            lib.ub_coexec_run.argtypes = [I, I, I, P, P]
            self.lib = lib
        self.cache = {}

    def _time(self, fn, reps: int) -> float:
        """Mean ms of fn(i) over reps calls (GPU timeline), after two warm-up calls."""
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def copy_GBs(self, nbytes: int = 1 << 30) -> float:
        """HBM streaming copy: bytes read + written per second."""
        if self.lib is None:
            return None
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        s = torch.cuda.current_stream().cuda_stream
        ms = self._time(lambda i: self.lib.ub_copy_run(src.data_ptr(), dst.data_ptr(), nbytes, s), 10)
        del src, dst
        return 2 * nbytes / (ms * 1e-3) / 1e9

    def mfma_TFLOPs(self, dtype: str) -> float:
        if self.lib is None:
            return None
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        blocks, iters = cus * 4, 1000
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        dt = 0 if dtype == "fp16" else 1
        ms = self._time(lambda i: self.lib.ub_mfma_run(dt, blocks, iters, out.data_ptr(), s), 5)
        return blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12

    def coexec_ns(self) -> dict:
        """ns per iteration of ub_coexec's four modes (one 8-wave workgroup per CU: per SIMD, two
        waves): MFMA only, VALU only, one MFMA wave beside one VALU wave, both in every wave.  The
        third equals the sum of the first two halves when a SIMD does not overlap one wave's
        MFMAs with another wave's VALU work."""
        if self.lib is None:
            return None
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        iters = 20000
        out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        names = ("mfma_waves", "valu_waves", "mfma_wave_beside_valu_wave", "mfma_and_valu_in_every_wave")
        res = {n: self._time(lambda i, m=m: self.lib.ub_coexec_run(m, cus, iters, out.data_ptr(), s), 3) * 1e6 / iters
               for m, n in enumerate(names)}
        res["sum_of_halves"] = (res["mfma_waves"] + res["valu_waves"]) / 2
        return res

    def gather_GBs(self, mode: int, shape: synth.SfaShape, sets) -> float:
        """Random-row gather of the workload's own K rows (every slot of every index list, one
        workgroup per list, rotating over the input sets): bytes moved per second.  mode 0: into
        an LDS ring by direct global->LDS loads; mode 1: into registers."""
        if self.lib is None:
            return None
        s = shape
        rb = s.Dk * 2
        if rb not in (256, 384, 1152):
            return None
        items = s.B * s.S1 * s.N2
        if s.layout == "BSND":
            per_batch, head_div = s.S1 * s.N2, 1
        else:
            per_batch, head_div = s.N2 * s.S1, s.S1
        st = [(x["k"], x["idx"]) for x in sets]
        k0 = st[0][0]
        kst = k0.stride()
        if s.layout == "BSND":
            batch_b, head_b, pitch = kst[0] * 2, kst[2] * 2, kst[1] * 2
        else:
            batch_b, head_b, pitch = kst[0] * 2, kst[1] * 2, kst[2] * 2
        threads = self.lib.ub_gather_reg_threads(rb)
        out = torch.empty(items * (threads if mode == 1 else 1), dtype=torch.int32, device="cuda")
        strm = torch.cuda.current_stream().cuda_stream
        for k, idx in st:  # every index lies in [0, S2): the rows the gather reads are inside k
            assert idx.is_contiguous() and k.stride() == kst and idx.numel() == items * s.topK

        def run(i):
            k, idx = st[i % len(st)]
            rc = self.lib.ub_gather_run(mode, rb, k.data_ptr(), idx.data_ptr(), items, s.topK, per_batch, head_div,
                                        s.N2, batch_b, head_b, pitch, out.data_ptr(), strm)
            if rc != 0:
                raise RuntimeError(f"ub_gather_run failed ({rc})")

        ms = self._time(run, 2 * len(st))
        return items * s.topK * rb / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------------------------
# top-K workloads

def topk_work(shape: synth.SfaShape, idx: torch.Tensor) -> dict:
    """Algorithmic work of one call: unmasked slots only; V rows counted only when V is not a
    view of K (then one gathered row serves both)."""
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
    return {"valid_slots": int(valid), "gathered_bytes": int(gathered),
            "alg_bytes": int(gathered + idx_bytes + qo_bytes), "flops": int(flops)}


def identity_indices(shape: synth.SfaShape) -> torch.Tensor:
    """Every key of the sequence in order (topK = S2): the dense operator through the sparse path."""
    s = shape
    ar = torch.arange(s.S2, dtype=torch.int32)
    if s.layout == "BSND":
        return ar.view(1, 1, 1, s.S2).expand(s.B, s.S1, s.N2, s.S2).contiguous()
    return ar.view(1, 1, 1, s.S2).expand(s.B, s.N2, s.S1, s.S2).contiguous()


class TopkSets:
    """n independent device-resident input sets of one workload, plus output and workspace, and
    one prepared library call per set (a single foreign call per step)."""

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
            self.sets.append({"q": inp["q"].to(dev), "k": k, "v": v, "idx": inp["idx"].to(dev),
                              "cpu": inp if r == 0 else None})
        s0, s = self.sets[0], shape
        need = api.workspace_bytes(s0["q"], s0["k"], s0["v"], s0["idx"], s.layout, s.causal)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.out = api.sparse_flash_attention(s0["q"], s0["k"], s0["v"], s0["idx"], s.scale_value, s.layout,
                                              s.causal, workspace=self.ws)
        torch.cuda.synchronize()
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


def _rate_topk(shape, inp, rows, threads, work_per_row, reps_max=200, budget_s=1.0):
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.sfa(inp["q"], inp["k"], inp["v"], inp["idx"], shape.scale_value, shape.layout, shape.causal,
                   rows=rows, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= reps_max:
            return len(rows) * reps * work_per_row / dt, len(rows) * reps, dt


def cpu_baseline(kind: str, unit: str, run_rows, nrows: int, work_total: float, budget_s: float = 10.0) -> dict:
    """Times the oracle on evenly spaced samples of the workload's query rows: all host threads
    for about budget_s, then one thread for about a quarter of that.  run_rows(rows, threads,
    budget) -> (work units per second, rows done, seconds); with budget 0 it makes one call.
    Two small calls first separate the oracle's fixed cost per call (input conversion) from its
    cost per row, so the timed sample is sized to the budget."""
    import oracle
    threads = oracle.default_threads()

    def size(nthreads, budget):
        r1 = np.linspace(0, nrows - 1, min(nrows, 16)).astype(np.int64)
        r2 = np.linspace(0, nrows - 1, min(nrows, 64)).astype(np.int64)
        t0 = time.perf_counter()
        run_rows(r1, nthreads, 0.0)
        t1 = time.perf_counter()
        run_rows(r2, nthreads, 0.0)
        t2 = time.perf_counter()
        per = max(((t2 - t1) - (t1 - t0)) / max(len(r2) - len(r1), 1), 1e-7)
        fixed = max((t1 - t0) - len(r1) * per, 0.0)
        n = int(min(nrows, max(len(r2), (budget - fixed) / per)))
        return np.linspace(0, nrows - 1, n).astype(np.int64)

    rows = size(threads, 0.8 * budget_s)
    rate, done, dt = run_rows(rows, threads, 0.8 * budget_s)
    rows1 = size(1, 0.2 * budget_s)
    rate1, done1, dt1 = run_rows(rows1, 1, 0.2 * budget_s)
    return {"value": rate, "unit": unit, "cores": threads, "kind": kind, "cpu_model": cpu_model(),
            "sample": f"{len(rows)} of {nrows} query rows (evenly spaced) of the timed inputs, {done} rows in "
                      f"{dt:.1f} s on {threads} threads; fp64 scalar C oracle",
            "single_thread_value": rate1,
            "single_thread_sample": f"{len(rows1)} rows, {done1} rows in {dt1:.1f} s on 1 thread",
            "workload_seconds_extrapolated": work_total / rate if rate > 0 else None,
            "workload_seconds_single_thread_extrapolated": work_total / rate1 if rate1 > 0 else None}


def bench_topk(name: str, steps: int, warmup: int, with_cpu: bool, dev: str, ceil: Ceilings = None,
               dense: bool = False) -> dict:
    """dense: the same workload with topK = S2 and identity indices (dense attention through the
    same kernels, the comparison baseline of the sparse form); two input sets rotate (its keys are
    L2 / MALL resident either way)."""
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
    t = time_steps(sets.step, steps, warmup)
    ms = t["ms_gpu_mean"]
    gbs = work["gathered_bytes"] / (t["ms_wall"] * 1e-3) / 1e9
    tflops_k = work["flops"] / (ms * 1e-3) / 1e12
    res = {"workload": name, "ms_per_step": t["ms_wall"], "timing_ms": t, "gathered_bytes": work["gathered_bytes"],
           "alg_bytes": work["alg_bytes"], "flops": work["flops"], "rotation_sets": len(sets.sets),
           "gathered_GBs": gbs, "TFLOPs": work["flops"] / (t["ms_wall"] * 1e-3) / 1e12,
           "gathered_GBs_gpu": work["gathered_bytes"] / (ms * 1e-3) / 1e9, "TFLOPs_gpu": tflops_k}
    # the bound: HBM for the decode problems (gathered bytes dominate), MFMA for prefill (its
    # gathered rows come from L2 / MALL: unique K is 25 MB), as the targets state them
    if name.startswith("gqa_prefill"):
        peak = MFMA_PEAK_TFLOPS[shape.dtype]
        res["roofline"] = {"bound": "mfma", "achieved": tflops_k, "peak": peak, "unit": "TFLOP/s",
                           "frac": tflops_k / peak, "traffic": measured_traffic(name)}
        res["metric_value"], res["unit"] = tflops_k, "TFLOP/s"
    else:
        ach = work["alg_bytes"] / (ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(name)}
        res["metric_value"], res["unit"] = res["gathered_GBs_gpu"], "GB/s"
    if ceil is not None and ceil.lib is not None and not dense:
        g_lds = ceil.gather_GBs(0, shape, sets.sets)
        g_reg = ceil.gather_GBs(1, shape, sets.sets)
        if g_lds:
            # the same rows (all slots, masked ones too) gathered by the microbenchmark: the
            # kernel's gathered-bytes rate against it
            res["roofline"]["ceiling"] = {"what": f"random {shape.Dk * 2}-byte row gather of the same index lists "
                                                  f"into LDS (direct loads), no compute",
                                          "GBs": g_lds, "GBs_registers": g_reg,
                                          "frac": res["gathered_GBs_gpu"] / g_lds}
    progress(f"{name}: {t['ms_wall'] * 1e3:.1f} us/step wall, {ms * 1e3:.1f} us GPU, median "
             f"{t['ms_step_median'] * 1e3:.1f} us, {gbs:.0f} GB/s gathered, {res['TFLOPs']:.1f} TFLOP/s")
    if with_cpu and not dense:
        progress(f"{name}: timing the fp64 CPU oracle on a sample")
        inp = sets.sets[0]["cpu"]
        nrows = shape.B * shape.S1 * shape.N1
        # the workload's work spread evenly over its query rows (sampled rows are evenly spaced)
        per_row = (work["gathered_bytes"] if res["unit"] == "GB/s" else work["flops"]) / nrows
        scale = 1e9 if res["unit"] == "GB/s" else 1e12

        def run_rows(rows, threads, budget):
            r, done, dt = _rate_topk(shape, inp, rows, threads, per_row, budget_s=budget)
            return r / scale, done, dt

        total = (work["gathered_bytes"] if res["unit"] == "GB/s" else work["flops"]) / scale
        res["cpu_baseline"] = cpu_baseline("oracle", res["unit"], run_rows, nrows, total)
    del sets
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------------------------
# block-sparse workloads

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


def bench_bsr(name: str, steps: int, warmup: int, dev: str, with_cpu: bool = False, ceil: Ceilings = None,
              mask_density: float = 0.0, fp8: str = "") -> dict:
    """mask_density > 0: a per-block mask whose elements are set with that probability.
    fp8 ("e4m3" / "e5m2"): FP8 q, k, v with per-head factors (the expansion to fp16 copies is
    part of every timed step)."""
    shape = synth.WORKLOADS[name]
    progress(f"{name}{' fp8 ' + fp8 if fp8 else ''}{' masked' if mask_density else ''}: generating inputs")
    sets = []
    for r in range(2):
        inp = synth.bsr_fp8_inputs(shape, fp8, fp8, seed=200 + r) if fp8 else synth.bsr_inputs(shape, seed=200 + r)
        if mask_density > 0:
            g = torch.Generator().manual_seed(300 + r)
            inp["mask"] = torch.rand((len(inp["indices"]), shape.R, shape.C), generator=g) < mask_density
        cpu = {k: v for k, v in inp.items()} if r == 0 else None
        sets.append({k: (v.to(dev) if k in ("q", "k", "v", "scale_q", "scale_k", "scale_v") else v)
                     for k, v in inp.items()})
        sets[-1]["cpu"] = cpu
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
    t = time_steps(step, steps, warmup)
    ms = t["ms_gpu_mean"]
    tflops_k = work["flops"] / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[shape.dtype]
    tag = name + ("_fp8_" + fp8 if fp8 else "") + (f"_masked_{mask_density}" if mask_density else "")
    res = {"workload": tag, "ms_per_step": t["ms_wall"], "timing_ms": t, "flops": work["flops"],
           "alg_bytes": work["alg_bytes"], "TFLOPs": work["flops"] / (t["ms_wall"] * 1e-3) / 1e12,
           "TFLOPs_gpu": tflops_k, "metric_value": tflops_k, "unit": "TFLOP/s",
           "roofline": {"bound": "mfma", "achieved": tflops_k, "peak": peak, "unit": "TFLOP/s",
                        "frac": tflops_k / peak,
                        "traffic": measured_traffic("bsr") if not fp8 and mask_density == 0 else None}}
    if ceil is not None and ceil.lib is not None:
        mf = ceil.mfma_TFLOPs(shape.dtype)
        if mf:
            res["roofline"]["ceiling"] = {"what": f"dense 32x32x16 {shape.dtype} MFMA, 16 waves per CU", "TFLOPs": mf,
                                          "frac": tflops_k / mf}
    if fp8:
        res["input_dtype"] = "fp8_" + fp8
        res["fp8_input_bytes"] = int(sum(sets[0][k].numel() for k in ("q", "k", "v")))
    progress(f"{tag}: {t['ms_wall'] * 1e3:.1f} us/step wall, {ms * 1e3:.1f} us GPU, {tflops_k:.1f} TFLOP/s")
    if with_cpu and not fp8 and mask_density == 0:
        import oracle
        progress(f"{tag}: timing the fp64 CPU oracle on a sample")
        cp = sets[0]["cpu"]
        nrows = shape.M * shape.Hq
        per_row = work["flops"] / nrows / 1e12  # every flat row of the workload has the same key count

        def run_rows(rows, threads, budget):
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.bsr(cp["q"], cp["k"], cp["v"], cp["indptr"], cp["indices"], shape.R, shape.C,
                           causal=shape.causal, rows=rows, nthreads=threads)
                reps += 1
                dt = time.perf_counter() - t0
                if dt >= budget or reps >= 200:
                    return len(rows) * reps * per_row / dt, len(rows) * reps, dt

        res["cpu_baseline"] = cpu_baseline("oracle", "TFLOP/s", run_rows, nrows, work["flops"] / 1e12)
    return res


def bench_dense_prefill(steps: int, warmup: int, dev: str, masked: bool = False) -> dict:
    """Dense attention at the GQA prefill shape through single_prefill_with_kv_cache: one call per
    batch of that workload (qo_len 1024, kv_len 4096, 64 query heads on 8 KV heads, Dqk 192, Dvo
    128 with value = key[..., :128], fp16), bottom-right causal or, with masked, the same causal
    pattern given as a custom mask.  Two input sets (one per batch) make a step."""
    w = synth.WORKLOADS["gqa_prefill"]
    qo, kv, Hq, Hkv, Dqk, Dvo = w.S1, w.S2, w.N1, w.N2, w.Dk, w.Dv
    progress(f"dense prefill{' (custom mask)' if masked else ''}: generating inputs")
    g = torch.Generator().manual_seed(500)
    dt = synth.DTYPES[w.dtype]
    sets = []
    for b in range(w.B):
        q = torch.randn((qo, Hq, Dqk), generator=g).to(dt).to(dev)
        k = torch.randn((kv, Hkv, Dqk), generator=g).to(dt).to(dev)
        sets.append((q, k, k[..., :Dvo]))
    mask = torch.tril(torch.ones((qo, kv), dtype=torch.bool), diagonal=kv - qo).to(dev) if masked else None
    out = torch.empty((qo, Hq, Dvo), dtype=dt, device=dev)
    need = binding.sfa_prefill_workspace_bytes(qo, kv, Hq, Hkv, Dqk, Dvo, masked)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    pairs = sum(min(kv, i + (kv - qo) + 1) for i in range(qo)) * w.B  # allowed (query row, key) pairs
    flops = pairs * Hq * 2 * (Dqk + Dvo)

    def step(i):
        for q, k, v in sets:
            api.single_prefill_with_kv_cache(q, k, v, custom_mask=mask, causal=not masked, out=out, workspace=ws)

    progress(f"dense prefill: timing {steps} steps")
    t = time_steps(step, steps, warmup)
    tflops_k = flops / (t["ms_gpu_mean"] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    progress(f"dense prefill: {t['ms_wall'] * 1e3:.1f} us/step, {tflops_k:.1f} TFLOP/s")
    return {"workload": "gqa_prefill_dense" + ("_custom_mask" if masked else ""), "ms_per_step": t["ms_wall"],
            "timing_ms": t, "flops": flops, "TFLOPs_gpu": tflops_k, "metric_value": tflops_k, "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": tflops_k, "peak": peak, "unit": "TFLOP/s",
                         "frac": tflops_k / peak, "traffic": None if masked else measured_traffic("dense")}}


def vbsr_work(shape: synth.VbsrShape, inp: dict) -> dict:
    """Algorithmic work of one variable block-sparse call: every allowed (query, key) pair of
    every query head, QK^T and PV; K and V rows loaded once per (block row, KV head)."""
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
    t = time_steps(step, steps, warmup)
    tflops_k = work["flops"] / (t["ms_gpu_mean"] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[shape.dtype]
    progress(f"vbsr: {t['ms_wall'] * 1e3:.1f} us/step, {tflops_k:.1f} TFLOP/s")
    return {"workload": "vbsr", "ms_per_step": t["ms_wall"], "timing_ms": t, "TFLOPs_gpu": tflops_k,
            "flops": work["flops"], "alg_bytes": work["alg_bytes"], "metric_value": tflops_k, "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": tflops_k, "peak": peak, "unit": "TFLOP/s",
                         "frac": tflops_k / peak, "traffic": measured_traffic("vbsr")}}


# ---------------------------------------------------------------------------------------------

def _round(x):
    if isinstance(x, float):
        return float(f"{x:.6g}")
    if isinstance(x, dict):
        return {k: _round(v) for k, v in x.items()}
    if isinstance(x, list):
        return [_round(v) for v in x]
    return x


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(synth.WORKLOADS) + ["vbsr", "dense"],
                    help="time this workload alone (for profiling runs); dense: the causal dense prefill at "
                         "the GQA prefill shape")
    ap.add_argument("--all", action="store_true",
                    help="also time the dense-through-sparse baseline, the masked / FP8 BSR calls and variable "
                         "block-sparse attention")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-ceilings", action="store_true",
                    help="also measure the ceiling microbenchmarks (libsfa_ubench.so) next to each workload")
    ap.add_argument("--ceilings", action="store_true", help="only run the ceiling microbenchmarks")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: there is no multi-GPU path in this library (asked for --gpus "
              f"{args.gpus})", file=sys.stderr)
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
    # The ceiling microbenchmarks load a second HIP library into the process; a default run with
    # them ended in a host segmentation fault whose cause is not established, so they run only
    # when asked for.
    ceil = Ceilings() if (args.with_ceilings or args.ceilings) else None
    if args.ceilings:
        if ceil is None or ceil.lib is None:
            print("libsfa_ubench.so is not built", file=sys.stderr)
            sys.exit(2)
        out = {"copy_GBs": ceil.copy_GBs(), "mfma_fp16_TFLOPs": ceil.mfma_TFLOPs("fp16"),
               "mfma_bf16_TFLOPs": ceil.mfma_TFLOPs("bf16"), "coexec_ns_per_iter": ceil.coexec_ns()}
        for name in ("gqa_decode", "mla_decode", "gqa_prefill"):
            shape = synth.WORKLOADS[name]
            probe = synth.sfa_inputs(shape, seed=100)
            n = n_rotation_sets(shape, topk_work(shape, probe["idx"]))
            del probe
            sets = TopkSets(shape, n, dev)
            out[name] = {"gather_lds_GBs": ceil.gather_GBs(0, shape, sets.sets),
                         "gather_registers_GBs": ceil.gather_GBs(1, shape, sets.sets)}
            del sets
            torch.cuda.empty_cache()
        print(json.dumps(_round(out)), flush=True)
        return
    with_cpu = not args.no_cpu_baseline
    if args.workload is not None:
        name = args.workload
        if name == "vbsr":
            res = bench_vbsr(args.steps, args.warmup, dev)
        elif name == "dense":
            res = bench_dense_prefill(args.steps, args.warmup, dev)
        elif name == "bsr":
            res = bench_bsr(name, args.steps, args.warmup, dev, with_cpu, ceil)
        else:
            res = bench_topk(name, args.steps, args.warmup, with_cpu, dev, ceil)
        shape = {"vbsr": synth.VBSR_WORKLOAD, "dense": synth.WORKLOADS["gqa_prefill"]}.get(name) or synth.WORKLOADS[name]
        print(json.dumps(_round({"metric": METRIC, "value": res["metric_value"], "unit": res["unit"], "n_gpus": 1,
                                 "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
                                 "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                                 "dtype": shape.dtype, "data": "synthetic",
                                 "config": ({"workload": "gqa_prefill_dense_causal", "calls": shape.B,
                                             "qo_len": shape.S1, "kv_len": shape.S2, "num_qo_heads": shape.N1,
                                             "num_kv_heads": shape.N2, "head_dim_qk": shape.Dk,
                                             "head_dim_vo": shape.Dv, "value": "key[..., :Dvo]"}
                                            if name == "dense" else {"workload": name, **dataclasses.asdict(shape)}),
                                 "roofline": res["roofline"], "cpu_baseline": res.get("cpu_baseline"),
                                 "detail": res})), flush=True)
        return

    main_res = bench_topk("gqa_decode", args.steps, args.warmup, with_cpu, dev, ceil)
    shape = synth.WORKLOADS["gqa_decode"]
    line = {
        "metric": METRIC,
        "value": main_res["gathered_GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded N(0,1) q/k, uniform top-K indices without replacement)",
        "config": {"workload": "gqa_decode", "B": shape.B, "S1": shape.S1, "S2": shape.S2, "N1": shape.N1,
                   "N2": shape.N2, "Dk": shape.Dk, "Dv": shape.Dv, "topK": shape.topK, "layout": shape.layout,
                   "causal": shape.causal, "parallelism": "single GPU"},
        "tflops": main_res["TFLOPs"],
        "frac_hbm_gathered": main_res["gathered_GBs"] / HBM_PEAK_GBS,
        "timing_ms": main_res["timing_ms"],
        "roofline": main_res["roofline"],
        "cpu_baseline": main_res.get("cpu_baseline"),
    }
    per = {"gqa_decode": {k: main_res[k] for k in ("metric_value", "unit", "ms_per_step", "timing_ms", "roofline",
                                                   "cpu_baseline", "gathered_GBs", "TFLOPs") if k in main_res}}
    for name in ("tiny", "mla_decode", "gqa_prefill"):
        r = bench_topk(name, args.steps, args.warmup, with_cpu, dev, ceil)
        per[name] = {k: r[k] for k in ("metric_value", "unit", "ms_per_step", "timing_ms", "roofline", "cpu_baseline",
                                       "gathered_GBs", "TFLOPs", "rotation_sets") if k in r}
    r = bench_bsr("bsr", args.steps, args.warmup, dev, with_cpu, ceil)
    per["bsr"] = {k: r[k] for k in ("metric_value", "unit", "ms_per_step", "timing_ms", "roofline", "cpu_baseline",
                                    "TFLOPs") if k in r}
    if ceil is not None and ceil.lib is not None:
        per["ceilings"] = {"copy_GBs": ceil.copy_GBs(), "mfma_fp16_TFLOPs": ceil.mfma_TFLOPs("fp16"),
                           "mfma_bf16_TFLOPs": ceil.mfma_TFLOPs("bf16")}
    if args.all:
        # the pages' complexity claim, O(S1 S2 D) -> O(S1 topK D), at the prefill shape: dense
        # attention through the dense entry point, and through the sparse kernels with every key
        # selected in order (identity indices)
        for masked in (False, True):
            r = bench_dense_prefill(args.steps, args.warmup, dev, masked=masked)
            r["sparse_speedup"] = r["ms_per_step"] / per["gqa_prefill"]["ms_per_step"]
            per[r["workload"]] = r
        r = bench_topk("gqa_prefill", args.steps, args.warmup, False, dev, dense=True)
        per["gqa_prefill_dense_gather"] = {k: r[k] for k in ("ms_per_step", "timing_ms", "TFLOPs_gpu")}
        per["gqa_prefill_dense_gather"]["sparse_speedup"] = r["ms_per_step"] / per["gqa_prefill"]["ms_per_step"]
        per["bsr_masked_0.5"] = bench_bsr("bsr", args.steps, args.warmup, dev, mask_density=0.5)
        per["bsr_fp8_e4m3"] = bench_bsr("bsr", args.steps, args.warmup, dev, fp8="e4m3")
        per["vbsr"] = bench_vbsr(args.steps, args.warmup, dev)
    line["per_config"] = per
    print(json.dumps(_round(line)), flush=True)


if __name__ == "__main__":
    main()
