"""Build the plain C client of the trellis C ABI (test infrastructure).

gcc compiles trellis_client.c against include/trellis.h and the HIP runtime's
C API and links the in-tree libtrellis.so (found at run time through an
rpath relative to the binary). Called by the repository's build entry point
after the library is built.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BINARY = os.path.join(HERE, "trellis_client")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "trellis_coded_bit_prefill_amd")
    tmp = BINARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           "-o", tmp, os.path.join(HERE, "trellis_client.c"),
           "-L", pkg, "-ltrellis", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../trellis_coded_bit_prefill_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    build(verbose=True)
