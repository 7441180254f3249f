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


@pytest.mark.skipif(not os.path.exists(_build.hipcc()), reason="hipcc not available")
def test_prefill_kernels_use_no_scratch_and_fit_four_waves_per_simd():
    asm = _device_asm()
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
