"""The compiled gfx950 assembly of every HIP source keeps the wait states that MFMA and LDS-DMA
hazards need, including around the instructions issued from inline assembly, which the compiler
does not see (the checker is `asm_hazards`). The checker itself is pinned on small hand-written
sequences and on copies of the real assembly with its guards removed.
"""
import importlib.util
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import asm_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "rswa_build_for_asm", os.path.join(ROOT, "windowed_attention_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm():
    """Device assembly of each HIP source, compiled with the library's own flags."""
    b = _build_module()
    if not shutil.which(b.HIPCC) and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc is not available")
    tmp = tempfile.mkdtemp(prefix="rswa_asm_")

    def one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [b.HIPCC, *b.HIP_FLAGS, *b.COMMON, *b.HIP_EXTRA.get(src, []), "--cuda-device-only",
               "-S", "-o", out, os.path.join(b.CSRC, src)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        with open(out) as f:
            return src, f.read()

    try:
        with ThreadPoolExecutor(len(b.HIP_SOURCES)) as ex:
            return dict(ex.map(one, b.HIP_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_sources_have_no_hazards(asm):
    for src, text in asm.items():
        assert H.check(text) == [], src


def test_checker_sees_the_hand_written_instructions(asm):
    """The parse finds the kernels and, in them, the inline-asm MFMAs and LDS DMAs."""
    funcs = H.parse(asm["prefill_bwd.hip"])
    ops = [i.op for f in funcs for b in f.blocks for i in b.instrs]
    assert any("dkdv_kernel" in f.name for f in funcs)
    assert ops.count("v_mfma_f32_32x32x16_bf16") > 100
    assert ops.count("global_load_lds_dwordx4") > 100
    text = asm["prefill_bwd.hip"]
    inline_mfma = sum(1 for blk in text.split(";;#ASMSTART")[1:]
                      if "v_mfma" in blk.split(";;#ASMEND")[0])
    assert inline_mfma > 0


def _drop_first(text, needle, after):
    """`text` without the first line equal to `needle` that follows a line containing `after`."""
    lines = text.splitlines()
    for i in range(1, len(lines)):
        if lines[i].strip() == needle and after in lines[i - 1]:
            return "\n".join(lines[:i] + lines[i + 1:])
    raise AssertionError(f"no {needle!r} after {after!r}")


def test_planted_missing_mfma_guard_is_found(asm):
    # the 12 wait states after the last MFMAs of the backward's score chains, taken out everywhere
    text = asm["prefill_bwd.hip"]
    n = text.count("\n\ts_nop 7\n\ts_nop 3\n")
    assert n > 0
    bad = text.replace("\n\ts_nop 7\n\ts_nop 3\n", "\n")
    found = H.check(bad)
    assert found and all("v_mfma" in x for x in found)


def test_planted_missing_m0_wait_is_found(asm):
    bad = _drop_first(asm["prefill.hip"], "s_nop 0", "s_mov_b32 m0")
    found = H.check(bad)
    assert len(found) == 1 and "M0 written" in found[0]


def _kernel(body):
    return f"k:\n{body}\n\ts_endpgm\n.Lfunc_end0:\n"


MFMA = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]"


@pytest.mark.parametrize("nop,bad", [(10, True), (11, False)])
def test_result_read_distance(nop, bad):
    text = _kernel(f"{MFMA}\n\ts_nop {nop}\n\tv_add_f32_e32 v20, v15, v15")
    assert bool(H.check(text)) == bad


def test_result_write_and_store_and_copy_are_accesses():
    for use in ("v_mov_b32_e32 v3, 0", "global_store_dword v20, v7, s[0:1]",
                "v_accvgpr_write_b32 a40, v15", "ds_write_b32 v20, v0"):
        assert H.check(_kernel(f"{MFMA}\n\ts_nop 7\n\t{use}")), use


def test_in_place_chain_needs_no_wait_but_other_uses_do():
    assert H.check(_kernel(f"{MFMA}\n{MFMA}\n\ts_nop 11\n\tv_add_f32_e32 v20, v1, v1")) == []
    other = "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], a[0:3], v[32:47]"  # reads v0..3 as A
    assert H.check(_kernel(f"{MFMA}\n{other}\n\ts_nop 11\n\ts_nop 11"))
    partial = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], 0"  # overwrites, no chain
    assert H.check(_kernel(f"{MFMA}\n{partial}\n\ts_nop 11\n\ts_nop 11"))


@pytest.mark.parametrize("between,bad", [("", True), ("\ts_nop 0\n", True),
                                         ("\ts_nop 1\n", False)])
def test_valu_write_before_mfma(between, bad):
    text = _kernel(f"\tv_mov_b32_e32 v5, 0\n{between}{MFMA}\n\ts_nop 11")
    assert bool(H.check(text)) == bad
    text = _kernel(f"\tv_accvgpr_write_b32 a2, v40\n{between}{MFMA}\n\ts_nop 11")  # B operand
    assert bool(H.check(text)) == bad


def test_load_result_before_mfma_is_not_a_wait_state_hazard():
    # a load's data is ordered by s_waitcnt, not by wait states
    assert H.check(_kernel(f"\tds_read_b128 v[16:19], v40\n\ts_waitcnt lgkmcnt(0)\n{MFMA}"
                           "\n\ts_nop 11")) == []


@pytest.mark.parametrize("between,bad", [("", True), ("\ts_nop 0\n", False),
                                         ("\tv_mov_b32_e32 v9, 0\n", False)])
def test_m0_write_before_lds_dma(between, bad):
    text = _kernel(f"\ts_mov_b32 m0, s4\n{between}\tglobal_load_lds_dwordx4 v2, s[6:7]")
    assert bool(H.check(text)) == bad


def test_hazards_are_followed_across_branches():
    # taken branch: the read sits at the target
    text = ("k:\n" + MFMA + "\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 15\n\ts_endpgm\n"
            ".LBB0_2:\n\tv_add_f32_e32 v20, v15, v15\n\ts_endpgm\n.Lfunc_end0:\n")
    assert H.check(text)
    # loop back edge: the MFMA at the end of the body, the read at the head
    text = ("k:\n\ts_mov_b32 s0, 0\n.LBB0_1:\n\tv_add_f32_e32 v20, v15, v15\n\ts_nop 3\n" + MFMA +
            "\n\ts_add_i32 s0, s0, 1\n\ts_cmp_lg_u32 s0, 8\n\ts_cbranch_scc1 .LBB0_1\n"
            "\ts_nop 15\n\ts_endpgm\n.Lfunc_end0:\n")
    found = H.check(text)
    assert found and "after 3 wait states" in found[0]
    # a write before the loop head reaches an MFMA at the head through the entry edge only
    text = ("k:\n\tv_mov_b32_e32 v5, 0\n.LBB0_1:\n" + MFMA + "\n\ts_nop 11\n\ts_nop 11\n"
            "\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n.Lfunc_end0:\n")
    assert len(H.check(text)) == 1


def test_unknown_mfma_opcode_is_reported():
    text = _kernel("\tv_mfma_f32_16x16x32_bf16 v[0:3], v[16:19], v[20:23], 0\n\ts_nop 15")
    assert "no wait-state figure" in H.check(text)[0]
