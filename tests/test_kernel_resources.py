"""Register and scratch use of the prefill kernels, from the compiler's own
resource report (device assembly of the library source, gfx950).

A prefill kernel that spills to scratch memory runs several times slower
(scratch is HBM) without failing any parity test, and one that needs more
than 128 VGPRs cannot keep four waves per SIMD. Compiling takes about a
minute on the CPU; no GPU is needed.
"""
import os
import re
import subprocess
import tempfile

import pytest

from trellis_coded_bit_prefill_amd import _build


def _device_asm() -> str:
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "trellis.s")
        cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(_build.ROOT, "include"),
               "-o", out, *_build.SOURCES]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(out) as f:
            return f.read()


needs_hipcc = pytest.mark.skipif(not os.path.exists(_build.hipcc()), reason="hipcc not available")


@pytest.fixture(scope="module")
def asm():
    return _device_asm()


def _kernels(asm):
    for blk in re.split(r"\n(?=_Z\S*:)", asm):
        name = blk.split(":", 1)[0]
        if "prefill_kernel" in name:
            yield name, blk


def _basic_blocks(blk):
    """Instruction mnemonics of each basic block of a kernel's assembly."""
    out, cur = [], None
    for line in blk.split("\n"):
        t = line.strip()
        if re.match(r"^(\.LBB\S+|; %bb\.\d+):", t):
            cur = []
            out.append(cur)
        elif cur is not None and t and not t.startswith((".", ";")):
            cur.append(t.split()[0])
    return out


@needs_hipcc
def test_prefill_kernels_use_no_scratch_and_fit_four_waves_per_simd(asm):
    # Each kernel's report follows its symbol: ".section ... <name>:" ...
    # "; ScratchSize: N" ... "; NumVgprs: N".
    blocks = re.split(r"\n(?=_Z\S*:)", asm)
    seen = 0
    for blk in blocks:
        name = blk.split(":", 1)[0]
        if "prefill_kernel" not in name:
            continue
        scratch = int(re.search(r"; ScratchSize: (\d+)", blk).group(1))
        vgprs = int(re.search(r"; TotalNumVgprs: (\d+)", blk).group(1))
        assert scratch == 0, f"{name} uses {scratch} bytes of scratch"
        assert vgprs <= 128, f"{name} uses {vgprs} VGPRs"
        seen += 1
    # k = 2, 3, 4 x (value, code table) + the pair table, each for one matrix
    # and for the fused gate and up projections
    assert seen == 14, f"expected 14 prefill kernels, found {seen}"


@needs_hipcc
def test_bf16_rounding_of_weights_uses_the_packed_convert(asm):
    # Every decoded weight is rounded from float32 to bf16 (round to nearest
    # even) before it enters the MFMA. gfx950 rounds two per instruction
    # (v_cvt_pk_bf16_f32); a software rounding (bias 0x7fff plus the lsb,
    # then a shift) would cost several VALU ops per weight.
    for name, blk in _kernels(asm):
        assert blk.count("v_cvt_pk_bf16_f32") >= 32, f"{name}: no packed bf16 convert"
        assert not re.search(r"v_add3_u32\S*\s.*0x7fff", blk), f"{name}: software bf16 rounding"


@needs_hipcc
def test_k4_unit_decode_instruction_budget(asm):
    # The k = 4 one-matrix kernels decode a unit (16 rows x 256 weights; per
    # lane 64 weights, 32 through the table and 32 through the hash on the
    # ALU) in one basic block with 8 MFMAs: 32 table gathers and 8 x reads
    # from LDS, and at most 292 VALU instructions (about 4.5 per weight:
    # hash, byte sum, fused multiply-add or scale, window extraction, one
    # packed convert per two weights). A regression here costs time on every
    # unit without failing a parity test.
    checked = 0
    for name, blk in _kernels(asm):
        if "prefill_kernelILi4ELi51ELi" not in name or "ELb0E" not in name:
            continue
        units = [b for b in _basic_blocks(blk) if b.count("v_mfma_f32_16x16x32_bf16") == 8
                 and b.count("v_sad_u8") == 32]
        assert units, f"{name}: no unit decode block found"
        for b in units:
            valu = sum(1 for m in b if m.startswith("v_"))
            assert valu <= 292, f"{name}: {valu} VALU instructions per unit"
            assert b.count("ds_read_b32") + b.count("ds_read_u16") == 32, f"{name}: table gathers"
            assert b.count("ds_read_b128") == 8, f"{name}: x reads"
        checked += 1
    assert checked == 2  # value table and code table


@needs_hipcc
def test_inline_asm_stores_wait_out_mfma_and_sgpr_hazards(asm):
    # The partial-tile stores are inline assembly, which the compiler's hazard
    # recognizer does not look into: without the padding, a store could read
    # an SGPR base address that a v_readlane (spill reload) wrote on the cycle
    # before, or an accumulator an MFMA is still writing. Every such store
    # (16 bytes, sc1) must follow at least 11 wait states of s_nop, directly
    # or behind the first store of a pair.
    seen = 0
    for name, blk in _kernels(asm):
        lines = [l.strip() for l in blk.split("\n") if l.strip() and not l.strip().startswith((";", "."))]
        for i, line in enumerate(lines):
            if not (line.startswith("global_store_dwordx4") and "sc1" in line):
                continue
            seen += 1
            k = i - 1
            if lines[k].startswith("global_store_dwordx4"):
                k -= 1
            waits = 0
            while k >= 0 and lines[k].startswith("s_nop"):
                waits += int(lines[k].split()[1]) + 1
                k -= 1
            assert waits >= 11, f"{name}: {line} after {waits} wait states"
    assert seen > 0
