"""The direct global->LDS loads are inline assembly, so the compiler's hazard checks do
not see them as memory instructions.  A vector-ALU write of an SGPR that a memory
instruction then reads as its scalar base needs five wait states in between; without
them the load may take a stale base and read from a wrong address.  This test compiles
every kernel source to gfx950 assembly (no GPU needed) and checks that no
global_load_lds_dwordx4 has a write of its base SGPRs within the five wait states
before it (s_nop N counts N+1)."""
import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from exact_io_aware_14_amd import build as B

KERNEL_SOURCES = ["fa_fwd_bf16.hip", "fa_bwd_bf16.hip", "fa_bwd_dq_bf16.hip"]
LOAD = re.compile(r"\s*global_load_lds_dwordx4 v\d+, s\[(\d+):(\d+)\]")


def _assembly(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    subprocess.run([B.hipcc(), *B.HIPCC_FLAGS, "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only", "-S",
                    os.path.join(B.CSRC, src), "-o", out], check=True, capture_output=True, text=True)
    return out


def _sgprs(operand: str) -> set:
    """SGPR names an operand covers: "s8" -> {s8}, "s[8:9]" -> {s8, s9}."""
    m = re.fullmatch(r"s(\d+)", operand)
    if m:
        return {operand}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", operand)
    if m:
        return {"s%d" % r for r in range(int(m.group(1)), int(m.group(2)) + 1)}
    return set()


def _hazards(lines):
    """(line, instruction) of every load whose base SGPRs are written in the five wait
    states before it."""
    bad = []
    for i, line in enumerate(lines):
        m = LOAD.match(line)
        if not m:
            continue
        base = {"s" + m.group(1), "s" + m.group(2)}
        k, ws = i - 1, 0
        while k >= 0 and ws < 5:
            t = lines[k].strip()
            k -= 1
            if not t or t.startswith(";") or t.startswith("."):
                continue
            parts = t.replace(",", " ").split()
            if parts[0] == "s_nop":
                ws += int(parts[1], 0) + 1
                continue
            if parts[0].startswith("v_") and len(parts) > 1 and _sgprs(parts[1]) & base:  # vector-ALU write
                bad.append((i, t))
                break
            ws += 1
    return bad


def test_hazard_scan_finds_a_planted_case():
    lines = ["\tv_readfirstlane_b32 s9, v3", "\tv_readfirstlane_b32 s8, v2",
             "\tglobal_load_lds_dwordx4 v1, s[8:9]"]
    assert len(_hazards(lines)) == 1
    assert _hazards(["\tv_readfirstlane_b32 s8, v2", "\ts_nop 4", "\tglobal_load_lds_dwordx4 v1, s[8:9]"]) == []
    # a vector instruction with a register-pair destination (a compare) counts as well
    assert len(_hazards(["\tv_cmp_gt_i32_e64 s[8:9], v1, v2", "\tglobal_load_lds_dwordx4 v1, s[8:9]"])) == 1
    assert _hazards(["\tv_readfirstlane_b32 s7, v2", "\tglobal_load_lds_dwordx4 v1, s[8:9]"]) == []
    # scalar-ALU writes of the base need no wait states
    assert _hazards(["\ts_add_u32 s8, s2, s4", "\ts_addc_u32 s9, s3, 0", "\tglobal_load_lds_dwordx4 v1, s[8:9]"]) == []


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()), reason="no hipcc")
def test_no_sgpr_base_hazard_before_lds_loads():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
            outs = list(ex.map(lambda s: _assembly(s, d), KERNEL_SOURCES))
        for src, out in zip(KERNEL_SOURCES, outs):
            lines = open(out).read().split("\n")
            assert any(LOAD.match(l) for l in lines), src
            bad = _hazards(lines)
            assert not bad, f"{src}: scalar base written right before a direct load: {bad[:3]}"
