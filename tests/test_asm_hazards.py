"""Inline-asm MFMAs and the per-block loops of the attention kernels, checked
in the compiled assembly.

An MFMA written as inline asm has accumulators the compiler cannot see as
MFMA results: the wait states around it, and the absence of spill code that
would move its accumulators, are then the kernel's own responsibility. The
checker below scans the gfx950 assembly of the source the library is built
from (same flags) for both; it is first shown to catch planted mistakes on
small hand-written listings. The current forward kernels issue their MFMAs
through builtins (the check then finds nothing to flag) and the fast-path
kernels must not spill.
"""

import os
import shutil
import subprocess

import pytest

import asm_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kernel(body: str) -> H.Kernel:
    text = "_ZN3sta12_GLOBAL__N_120sta_attention_kernelTEST:\n" + body + "\n.Lfunc_end0:\n"
    ks = H.parse(text)
    assert len(ks) == 1
    return ks[0]


ASM_MFMA = "\t;;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[12:15], a[0:15]\n\t;;#ASMEND\n"


def test_checker_flags_early_accumulator_read():
    bad = _kernel(ASM_MFMA + "\ts_nop 7\n\tv_accvgpr_read_b32 v0, a3\n\ts_endpgm\n")
    assert len(H.check_result_reads(bad)) == 1
    good = _kernel(ASM_MFMA + "\ts_nop 15\n\ts_nop 1\n\tv_accvgpr_read_b32 v0, a3\n\ts_endpgm\n")
    assert H.check_result_reads(good) == []


def test_checker_flags_spill_store_of_accumulator():
    bad = _kernel(ASM_MFMA + "\tscratch_store_dwordx4 off, a[0:3], off offset:400\n\ts_endpgm\n")
    assert len(H.check_result_reads(bad)) == 1


def test_checker_allows_accumulation_chain_and_other_accumulators():
    other = ASM_MFMA.replace("a[0:15], v[8:11], v[12:15], a[0:15]", "a[16:31], v[8:11], v[12:15], a[16:31]")
    k = _kernel(ASM_MFMA + ASM_MFMA + other + "\ts_endpgm\n")
    assert H.check_result_reads(k) == []
    # an MFMA that reads the accumulator as a plain operand is not a chain
    k = _kernel(ASM_MFMA + ASM_MFMA.replace("a[0:15], v[8:11], v[12:15], a[0:15]",
                                            "a[16:31], v[8:11], v[12:15], a[0:15]") + "\ts_endpgm\n")
    assert len(H.check_result_reads(k)) == 1


def test_checker_follows_branches():
    body = (ASM_MFMA + "\ts_cbranch_scc1 .LBB0_2\n\ts_nop 15\n\ts_nop 15\n.LBB0_2:\n"
            "\tv_accvgpr_read_b32 v0, a0\n\ts_endpgm\n")
    assert len(H.check_result_reads(_kernel(body))) == 1  # the taken branch reaches the read early


def test_checker_flags_operand_written_just_before():
    bad = _kernel("\tv_cvt_pk_bf16_f32 v13, v1, v2\n" + ASM_MFMA + "\ts_endpgm\n")
    assert len(H.check_operand_writes(bad)) == 1
    bad2 = _kernel("\tv_cvt_pk_bf16_f32 v13, v1, v2\n\ts_nop 0\n" + ASM_MFMA + "\ts_endpgm\n")
    assert len(H.check_operand_writes(bad2)) == 1
    good = _kernel("\tv_cvt_pk_bf16_f32 v13, v1, v2\n\ts_nop 1\n" + ASM_MFMA + "\ts_endpgm\n")
    assert H.check_operand_writes(good) == []
    unrelated = _kernel("\tv_cvt_pk_bf16_f32 v20, v1, v2\n" + ASM_MFMA + "\ts_endpgm\n")
    assert H.check_operand_writes(unrelated) == []


def _compile_asm(tmp_path_factory, src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from block_sparse_sliding_amd import build as B

    out = tmp_path_factory.mktemp("asm") / src.replace(".hip", ".s")
    cmd = [hipcc, *B.HIPCC_FLAGS, *B.EXTRA_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    return out.read_text()


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    return _compile_asm(tmp_path_factory, "sta_attention.hip")


@pytest.fixture(scope="module")
def backward_asm(tmp_path_factory):
    return _compile_asm(tmp_path_factory, "sta_backward.hip")


def test_loop_checker_flags_waits_and_spills():
    loop = ("\ts_mov_b32 s0, 0\n.LBB0_1:\n" + ASM_MFMA * 40 + "{}\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    assert H.check_block_loops(_kernel(loop.format(""))) == []
    asm_wait = "\t;;#ASMSTART\n\ts_waitcnt vmcnt(0)\n\t;;#ASMEND\n"
    assert H.check_block_loops(_kernel(loop.format(asm_wait))) == []
    assert len(H.check_block_loops(_kernel(loop.format("\ts_waitcnt vmcnt(3)\n")))) == 1
    assert len(H.check_block_loops(_kernel(loop.format("\tscratch_load_dword v0, off, off\n")))) == 1
    # a loop with few MFMAs (not a block loop) and an outer loop around the block loop are not checked
    assert H.check_block_loops(_kernel(loop.format("\ts_waitcnt vmcnt(3)\n")), min_mfma=64) == []
    outer = ".LBB0_0:\n\ts_waitcnt vmcnt(1)\n" + loop.format("").replace("\ts_endpgm\n", "\ts_cbranch_scc0 .LBB0_0\n\ts_endpgm\n")
    assert H.check_block_loops(_kernel(outer)) == []


def test_forward_kernels_no_asm_hazards(attention_asm):
    """No inline-asm MFMA of the forward kernels (there may be none) has an
    accumulator touched or an operand written too early; the kernels for
    tile-multiple videos (the fast path) spill nothing."""
    kernels = H.parse(attention_asm)
    names = sorted(k.name for k in kernels)
    # D in {64, 128} x (tile-multiple video, partial tiles, Hilbert units, square units,
    # square units with partial tiles)
    assert len(kernels) == 10, names
    for k in kernels:
        assert len(k.instrs) > 1000, k.name
        problems = H.check_result_reads(k) + H.check_operand_writes(k)
        assert problems == [], "\n".join(problems[:10])
        if "ELb0ELi0E" in k.name:  # PAD = false, single-tile units
            assert k.scratch == 0, f"{k.name}: {k.scratch} bytes of scratch per lane"
            assert k.vgpr_spills == 0, f"{k.name}: {k.vgpr_spills} VGPR spills"


def test_block_loops_wait_only_on_their_own_loads(attention_asm, backward_asm):
    """No spill reload and no compiler-placed vector-memory wait inside any
    per-block loop of the forward (all unit kinds), dq and dk/dv kernels: such a wait
    would also count the next block's LDS-DMA in flight."""
    kernels = H.parse(attention_asm) + H.parse(backward_asm, name_filter="bwd_d")
    names = sorted(k.name for k in kernels)
    assert len(kernels) == 10 + 6 + 6, names  # forward; dq and dk/dv (single tiles, squares)
    for k in kernels:
        assert H.innermost_loops(k), k.name
        problems = H.check_block_loops(k)
        assert problems == [], "\n".join(problems[:10])
