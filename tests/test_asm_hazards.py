"""Static check of the gfx950 assembly of the HIP kernels (CPU only).

Inline asm that writes SCC (for example the exec-masked y store, whose
s_and_b64 sets SCC) must declare the clobber.  Otherwise the compiler may
keep a carry or compare result in SCC across the statement; a 64-bit scalar
pointer increment split around it (s_add_u32 ... asm ... s_addc_u32) then
takes a wrong carry and moves a tile pointer by 2^32 bytes.  This test
compiles every kernel source to device assembly and fails if any SCC value
is live across an inline-asm block that writes SCC.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mamba_ssd_chunked_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SCC_DEF = re.compile(r"^(s_cmp|s_bitcmp|s_and_|s_or_|s_xor_|s_andn2_|s_orn2_|s_nand|s_nor|s_xnor|"
                     r"s_add_u32|s_sub_u32|s_add_i32|s_sub_i32|s_addc|s_subb|s_lshl|s_lshr|s_ashr|"
                     r"s_bfe|s_abs|s_not|s_min|s_max)")
SCC_USE = re.compile(r"^(s_cbranch_scc|s_cselect|s_addc|s_subb|s_cmov)")


def _op(line):
    t = line.strip().split()
    if not t or t[0].startswith(";") or t[0].startswith("."):
        return None
    return t[0]


def scc_live_across_asm(lines):
    """(line, text) of SCC reads whose value was set before an SCC-writing
    inline-asm block and not redefined after it."""
    hits = []
    i = 0
    while i < len(lines):
        if "ASMSTART" in lines[i]:
            j = i + 1
            writes = False
            while j < len(lines) and "ASMEND" not in lines[j]:
                op = _op(lines[j])
                if op and SCC_DEF.match(op):
                    writes = True
                j += 1
            if writes:
                for k in range(j + 1, min(j + 200, len(lines))):
                    if lines[k].startswith(".LBB"):
                        break
                    op = _op(lines[k])
                    if not op:
                        continue
                    if SCC_USE.match(op):
                        hits.append((k + 1, lines[k].strip()))
                        break
                    if SCC_DEF.match(op) or op.startswith("s_cbranch") or op.startswith("s_branch") \
                            or op == "s_endpgm":
                        break
            i = j
        i += 1
    return hits


def test_checker_flags_split_carry():
    """The checker itself: a carry split around an SCC-writing asm block is
    flagged, a carry kept together after it is not."""
    bad = ["\ts_add_u32 s86, s86, s48", "\t;;#ASMSTART", "\ts_and_b64 exec, exec, s[34:35]",
           "\tglobal_store_dwordx2 v79, v[0:1], s[30:31]", "\t;;#ASMEND", "\ts_addc_u32 s87, s87, s49"]
    good = ["\t;;#ASMSTART", "\ts_and_b64 exec, exec, s[34:35]", "\t;;#ASMEND",
            "\ts_add_u32 s86, s86, s48", "\ts_addc_u32 s87, s87, s49"]
    barrier = ["\ts_add_u32 s86, s86, s48", "\t;;#ASMSTART", "\ts_waitcnt lgkmcnt(0)", "\ts_barrier",
               "\t;;#ASMEND", "\ts_addc_u32 s87, s87, s49"]
    assert len(scc_live_across_asm(bad)) == 1
    assert scc_live_across_asm(good) == []
    assert scc_live_across_asm(barrier) == []


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_scc_live_across_inline_asm(src):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-o", out, os.path.join(CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = open(out).read().split("\n")
    hits = scc_live_across_asm(lines)
    assert hits == [], hits[:5]
