"""Wait states before every LDS-DMA load in the compiled kernels (CPU: hipcc cross-compiles).

The global -> LDS loads (`global_load_lds_dword[x4]`) are issued from inline asm, where the
compiler does not pad the hazards before them. The ISA requires wait states between writing an
SGPR and a vector-memory instruction reading it: 5 after a VALU write (v_readfirstlane, v_readlane
restoring a spilled SGPR, a carry-out), 1 after a SALU write of M0. A load with fewer can take the
register's previous value as its base address or LDS destination. These tests compile every
top-K instantiation unit and the ceiling microbenchmarks to assembly and check every load site.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_attention_13_amd import build

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_attention_13_amd")

# VALU opcodes whose second operand is an SGPR destination (carry-out or a scalar result)
_SDST2 = ("v_add_co", "v_sub_co", "v_subrev_co", "v_addc_co", "v_subb_co", "v_subbrev_co", "v_mad_u64_u32",
          "v_mad_i64_i32", "v_div_scale")


def _sgprs(tok: str) -> set:
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+", tok):
        return {tok}
    if tok == "m0":
        return {"m0"}
    return set()


def _valu_sgpr_writes(op: str, ops: list) -> set:
    if not op.startswith("v_") or not ops:
        return set()
    if op.startswith("v_cmp") and op.endswith("_e32"):
        return set()  # writes VCC, which no load reads
    w = _sgprs(ops[0])  # v_readfirstlane / v_readlane / v_cmp_e64 destinations
    if op.startswith(_SDST2) and len(ops) > 1:
        w |= _sgprs(ops[1])
    return w


def dma_hazards(asm_text: str) -> tuple:
    """(load sites, [(function, writer, wait states, load)]) for the LDS-DMA loads whose SGPR
    operands (M0 and a scalar base) were written too few wait states before."""
    sites, bad = 0, []
    fn, window = None, []
    for line in asm_text.splitlines():
        if re.match(r"^[A-Za-z_][\w.$]*:", line):
            fn, window = line.split(":")[0], []
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        op = parts[0]
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        if op.startswith("global_load_lds"):
            sites += 1
            reads = {"m0"}
            for o in ops[1:]:
                reads |= _sgprs(o)
            ws = 0
            for pop, pops in reversed(window):
                if pop == "s_nop":
                    ws += int(pops[0], 0) + 1
                    continue
                if _valu_sgpr_writes(pop, pops) & reads and ws < 5:
                    bad.append((fn, f"{pop} {', '.join(pops)}", ws, t))
                    break
                if pop.startswith("s_") and pops and pops[0] == "m0" and ws < 1:
                    bad.append((fn, f"{pop} {', '.join(pops)}", ws, t))
                    break
                ws += 1
                if ws >= 5:
                    break
        window = (window + [(op, ops)])[-8:]
    return sites, bad


def test_checker_flags_planted_hazards():
    planted = """k:
\tv_readfirstlane_b32 s17, v14
\tv_readfirstlane_b32 s16, v15
\ts_nop 0
\tglobal_load_lds_dwordx4 v18, s[16:17]
\ts_mov_b32 m0, s3
\tglobal_load_lds_dword v[2:3], off
\tv_mad_u64_u32 v[4:5], s[8:9], v1, s0, v[2:3]
\ts_nop 2
\tglobal_load_lds_dwordx4 v6, s[8:9]
"""
    sites, bad = dma_hazards(planted)
    assert sites == 3 and len(bad) == 3, bad
    padded = planted.replace("\ts_nop 0\n", "\ts_nop 4\n").replace("\ts_nop 2\n", "\ts_nop 4\n").replace(
        "\tglobal_load_lds_dword v[2:3], off", "\ts_nop 0\n\tglobal_load_lds_dword v[2:3], off")
    sites, bad = dma_hazards(padded)
    assert sites == 3 and bad == [], bad
    # an unrelated SGPR written just before, and a VGPR address written just before, are fine
    sites, bad = dma_hazards("k:\n\tv_readfirstlane_b32 s20, v1\n\tv_mov_b32 v6, 0\n\ts_nop 0\n"
                             "\tglobal_load_lds_dwordx4 v6, s[16:17]\n")
    assert sites == 1 and bad == []


def _assembly(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = list(build.FLAGS)
    r = subprocess.run([build.hipcc()] + flags + ["-S", "--offload-device-only", src, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc is not available")
def test_compiled_dma_loads_have_their_wait_states():
    # every instantiation unit (the hazard depends on each kernel's register allocation) and the
    # microbenchmarks
    units = sorted(os.path.join(CSRC, "csrc", f) for f in os.listdir(os.path.join(CSRC, "csrc"))
                   if f.startswith("topk_inst_") and f.endswith(".hip"))
    units.append(os.path.join(CSRC, "ubench", "ubench.hip"))
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(4) as ex:
        texts = list(ex.map(lambda u: _assembly(u, d), units))
    for unit, text in zip(units, texts):
        sites, bad = dma_hazards(text)
        assert sites > 0, unit
        assert bad == [], (os.path.basename(unit), bad[:5])
