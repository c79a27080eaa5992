"""Every gfx950 kernel that issues loads through inline assembly keeps their
destination registers untouched until the explicit wait that retires them.

Compiles the kernel sources to assembly with the library's own flags (host-only,
no GPU needed) and runs the control-flow walk in asm_hazards.py.  A planted
mistake (a register reused while its load is in flight) must be caught.
"""
import os
import shutil
import subprocess

import pytest

import asm_hazards as ah

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not on PATH")

PLANTED = """\
_Z6plantedv:
\t;;#ASMSTART
\tglobal_load_dwordx4 v[10:13], v[2:3], off
\t;;#ASMEND
\t;;#ASMSTART
\tglobal_load_dwordx4 v[14:17], v[4:5], off
\t;;#ASMEND
\ts_waitcnt vmcnt(1)
\tv_mov_b32 v0, v10
.LBB0_1:
\tv_add_u32_e32 v14, 1, v1
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""


def test_checker_catches_planted_reuse():
    k = ah.split_kernels(PLANTED)["_Z6plantedv"]
    hz = ah.kernel_hazards(k)
    # v10 is read after its load retired (fine); v14 is overwritten while in flight
    assert [h[0] for h in hz] == ["v_add_u32_e32 v14, 1, v1"]


def test_checker_lds_loads_write_no_register():
    text = """\
_Z3dmav:
\t;;#ASMSTART
\ts_mov_b32 m0, s4
\tglobal_load_lds_dwordx4 v[2:3], off
\t;;#ASMEND
\tv_add_u32_e32 v2, 16, v2
\ts_mov_b32 m0, s5
\ts_endpgm
.Lfunc_end2:
"""
    k = ah.split_kernels(text)["_Z3dmav"]
    assert ah.kernel_hazards(k) == []          # the address register may be reused at once
    assert ah.m0_writers(k) == ["s_mov_b32 m0, s5"]


def test_checker_follows_loop_back_edges():
    text = """\
_Z4loopv:
.LBB1_1:
\t;;#ASMSTART
\tglobal_load_dwordx2 v[20:21], v[2:3], off
\t;;#ASMEND
\ts_waitcnt vmcnt(1)
\tv_mov_b32 v5, v20
\ts_cbranch_scc1 .LBB1_1
\ts_endpgm
.Lfunc_end1:
"""
    # vmcnt(1) leaves the load just issued in flight, so v20 is read too early; the
    # walk must also carry the pending load around the back edge without looping
    hz = ah.kernel_hazards(ah.split_kernels(text)["_Z4loopv"])
    assert any("v_mov_b32 v5, v20" == h[0] for h in hz)


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    from speculative_decoding_attn_amd import build as b
    out = tmp_path_factory.mktemp("asm")
    texts = {}
    for src in ("lm_head.hip", "tree_attn.hip"):
        dst = out / src.replace(".hip", ".s")
        subprocess.run(["hipcc", *b.flags(), "--cuda-device-only", "-S",
                        os.path.join(b.CSRC, src), "-o", str(dst)], check=True)
        texts[src] = dst.read_text()
    return texts


@pytest.mark.parametrize("src", ["lm_head.hip", "tree_attn.hip"])
def test_inline_asm_loads_are_safe(kernel_asm, src):
    kernels = ah.split_kernels(kernel_asm[src])
    assert kernels
    problems = []
    for name, lines in kernels.items():
        if not ah.has_asm_loads(lines):
            continue
        if ah.indirect_indexing(lines):
            problems.append((name, "indirect register indexing"))
        if any('global_load_lds' in ln for ln in lines):
            problems += [(name, "compiler use of m0", x) for x in ah.m0_writers(lines)[:3]]
        for ins, _ in ah.kernel_hazards(lines)[:3]:
            problems.append((name, ins))
    assert not problems, problems
