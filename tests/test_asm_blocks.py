"""Host-side checks of the generated inline-asm blocks of the bf16 grouped GEMM.

The blocks in mfma_steps.inc are written by gen_mfma_steps.py; a stale file
or a block whose clobber list misses a register it writes would miscompile
silently (the compiler keeps values in M0 and SCC across asm statements it
believes leave them alone).
"""
import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "top_routing_expert_02_amd", "csrc")
INC = os.path.join(CSRC, "mfma_steps.inc")

# scalar ALU instructions that write SCC (those the blocks could use)
SCC_WRITERS = re.compile(r"\b(s_add_u32|s_add_i32|s_sub_u32|s_sub_i32|s_addc_u32|s_subb_u32|"
                         r"s_cmp_\w+|s_and_b\d+|s_or_b\d+|s_xor_b\d+|s_lshl_b\d+|s_lshr_b\d+)\b")


def split_asm(stmt):
    """(instruction text, operand and clobber sections) of one asm statement:
    the sections start at the first line that begins with a colon."""
    parts = re.split(r"\n\s*:", stmt)
    return parts[0], parts[1:]


def asm_blocks(text):
    """(body, clobbers) of every asm volatile(...) statement."""
    out = []
    for m in re.finditer(r"asm volatile\((.*?)\);", text, re.S):
        body, sections = split_asm(m.group(1))
        out.append((body, sections[2] if len(sections) >= 3 else ""))
    return out


def test_generated_file_is_current(tmp_path):
    spec = importlib.util.spec_from_file_location("gen_mfma_steps", os.path.join(CSRC, "gen_mfma_steps.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    parts = []
    for tm, tn in gen.SHAPES:
        parts.append(gen.emit(tm, tn))
    parts.append(gen.emit_w_stage())
    body = "".join(parts)
    with open(INC) as f:
        current = f.read()
    assert body in current, "mfma_steps.inc is stale: rerun gen_mfma_steps.py"


def test_blocks_declare_what_they_write():
    with open(INC) as f:
        text = f.read()
    blocks = asm_blocks(text)
    assert len(blocks) >= 4 * 5
    for body, clobbers in blocks:
        if "m0" in body:
            assert '"m0"' in clobbers, body[:120]
        if SCC_WRITERS.search(body):
            assert '"scc"' in clobbers, body[:120]


@pytest.mark.parametrize("tm", [1, 2, 3, 4])
def test_dma_halves_cover_each_load_once(tm):
    """The two halves of a stage's LDS-DMA loads issue every 1 KiB block of
    the stage exactly once: 2 TM token blocks from the token base, then 8
    weight blocks from the weight base."""
    with open(INC) as f:
        text = f.read()
    loads = []
    for half in (0, 1):
        m = re.search(r"void step_dma%d_%dx4\(.*?asm volatile\((.*?)\);" % (half, tm), text, re.S)
        assert m, (half, tm)
        body, _ = split_asm(m.group(1))
        nacc, nfrag = 4 * tm, tm + 4
        # operand numbers: acc, next fragments, current fragments, ta, wa,
        # vo[2 TM + 8], la, lb, ga, gw
        vo0 = nacc + nfrag + nfrag + 2
        la, lb, ga, gw = vo0 + 2 * tm + 8, vo0 + 2 * tm + 9, vo0 + 2 * tm + 10, vo0 + 2 * tm + 11
        m0 = None
        for line in re.findall(r'"([^"]*?)(?:\\n\\t)?"', body):
            mm = re.match(r"s_add_u32 m0, %(\d+), 0x([0-9a-f]+)", line)
            if mm:
                m0 = (int(mm.group(1)), int(mm.group(2), 16))
            mm = re.match(r"global_load_lds_dwordx4 %(\d+), %(\d+)", line)
            if mm:
                vo, g = int(mm.group(1)), int(mm.group(2))
                assert m0 is not None
                loads.append((vo - vo0, m0[0], m0[1], g))
                m0 = None
    na = 2 * tm
    expect = [(b, la, b * 0x400, ga) for b in range(na)] + \
             [(na + b, lb, b * 0x400, gw) for b in range(8)]
    assert sorted(loads) == sorted(expect)
