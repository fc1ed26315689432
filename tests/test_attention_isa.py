"""Checks on the generated gfx950 ISA of the verify-attention and verify-linear
kernels, the ones that use the LDS-DMA ring (CPU only: hipcc cross-compiles the
device code to assembly).

* Every LDS-DMA load is issued by the inline-asm sequence that saves M0, sets it, loads
  and restores it, so the asm never changes M0 behind the compiler's back.
* No transposed V read (ds_read_b64_tr_b16) or K read (ds_read_b128) waits for every
  vector load in flight: between a barrier and the LDS reads of a tile there is no
  s_waitcnt vmcnt(0), which would drain the DMA ring on every tile.
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_sd_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verification_sd_amd", "csrc")
# translation unit, kernels that use the DMA ring, minimum instantiations
UNITS = {
    "attention": ("attention.hip", r"verify_attn_(?:main|wide)", 8),
    "gemm": ("gemm.hip", r"verify_gemmI", 4),
}


def _compile(tmp_path_factory, unit):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    fname, pattern, least = UNITS[unit]
    out = tmp_path_factory.mktemp("isa") / (unit + ".s")
    cmd = [cc, *B.COMMON_FLAGS, *B.DEVICE_FLAGS, *B.FILE_FLAGS.get(fname, []), "--cuda-device-only",
           "-S", os.path.join(CSRC, fname), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    text = out.read_text()
    found = {}
    for m in re.finditer(r"^(_Z\w*" + pattern + r"\w*):[^\n]*\n(.*?)^\.Lfunc_end\d+:", text, re.M | re.S):
        found[m.group(1)] = [l.strip() for l in m.group(2).split("\n")]
    assert len(found) >= least, f"expected every instantiation of the {unit} kernels"
    return found


@pytest.fixture(scope="module")
def attention_kernels(tmp_path_factory):
    return _compile(tmp_path_factory, "attention")


@pytest.fixture(scope="module")
def gemm_kernels(tmp_path_factory):
    return _compile(tmp_path_factory, "gemm")


@pytest.fixture(params=["attention", "gemm"])
def kernels(request):
    return request.getfixturevalue(request.param + "_kernels")


def _instrs(lines):
    return [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]


def test_dma_sequence_saves_and_restores_m0(kernels):
    """Every LDS-DMA load sits in the inline-asm sequence that saves M0, sets it,
    waits one state, loads, and restores M0 from the saved SGPR: the asm leaves
    M0 as it found it, whatever the compiler keeps there."""
    for name, lines in kernels.items():
        ins = _instrs(lines)
        n = 0
        for i, l in enumerate(ins):
            if not l.startswith("global_load_lds_dwordx4"):
                continue
            n += 1
            save = re.match(r"s_mov_b32 (s\d+|vcc_lo|vcc_hi), m0$", ins[i - 3])
            assert save and re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", ins[i - 2]) and ins[i - 1] == "s_nop 0", \
                (name, ins[i - 3:i + 1])
            assert ins[i + 1] == f"s_mov_b32 m0, {save.group(1)}", (name, ins[i - 3:i + 2])
        assert n > 0, name


def test_no_full_vmem_drain_before_tile_reads(kernels):
    """No K/V tile read (ds_read_b128 / ds_read_b64_tr_b16) is preceded, within its
    basic block, by an s_waitcnt vmcnt(0): the compiler must not drain the DMA ring
    in front of the tile reads (the ring's own waits are explicit and counted)."""
    for name, lines in kernels.items():
        block = []
        for l in lines:
            if not l or l.startswith(";"):
                continue
            if l.endswith(":") or l.startswith(".LBB") or l.startswith("s_barrier"):
                block = []
                continue
            if l.startswith(("ds_read_b64_tr_b16", "ds_read_b128")):
                assert not any(re.match(r"s_waitcnt .*vmcnt\(0\)", x) for x in block), (name, l)
            block.append(l)


def test_dma_base_is_not_sign_extended(kernels):
    """The scalar DMA base is built from two readfirstlane words; the low word must be
    zero-extended (a sign-extending s_bfe_i64 there corrupts addresses whose low word
    has bit 31 set)."""
    for name, lines in kernels.items():
        assert not any(l.startswith("s_bfe_i64") for l in _instrs(lines)), name


def test_no_scratch_in_tile_loop(kernels):
    """No register spills: scratch loads and stores are vector-memory operations and
    would count against the vmcnt waits that pace the LDS-DMA ring."""
    for name, lines in kernels.items():
        assert not any(l.startswith(("scratch_", "buffer_store", "buffer_load")) for l in _instrs(lines)), name
