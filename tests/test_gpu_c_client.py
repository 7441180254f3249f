"""The C ABI from a plain C program: no Python or torch in the process.

tests/c_client/trellis_client (built by the repository's build entry point)
allocates device memory with hipMalloc, calls trellis_prefill and
trellis_decode on a stream of its own, calls trellis_prefill with an
unsupported batch, and writes the results back. The decoded weights must
match the CPU oracle bit for bit and the layer outputs must meet the
tolerance of the other parity tests; the rejected call must return
TRELLIS_E_M.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests.c_client.build import BINARY
from tests.helpers import assert_prefill_close
from workloads import generate

pytestmark = pytest.mark.gpu

OK, E_M = 0, -2


@pytest.fixture(scope="module", autouse=True)
def need_gpu_and_client():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BINARY), f"{BINARY} is not built; run the build entry point"


@pytest.mark.parametrize("m,k,n,bits", [(5, 512, 256, 2), (8, 1280, 324, 3), (15, 17408, 132, 4)])
def test_c_client(m, k, n, bits):
    print(f"C client m={m} k={k} n={n} bits={bits}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=9100 + m + bits)
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            f.write(np.array([m, k, n, bits], dtype=np.int32).tobytes())
            f.write(np.ascontiguousarray(x, dtype=np.uint16).tobytes())
            f.write(np.ascontiguousarray(codes, dtype=np.uint32).tobytes())
            f.write(np.ascontiguousarray(scales, dtype=np.uint16).tobytes())
        run = subprocess.run([BINARY, fin, fout], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0, run.stdout + run.stderr
        raw = open(fout, "rb").read()
    res = np.frombuffer(raw[:16], dtype=np.int32)
    out = np.frombuffer(raw[16:16 + 2 * m * n], dtype=np.uint16).reshape(m, n)
    w = np.frombuffer(raw[16 + 2 * m * n:], dtype=np.uint16).reshape(n, k)
    assert res.tolist() == [OK, OK, E_M, 1], run.stdout
    assert np.array_equal(w, oracle.decode(codes, scales, k, bits))
    y, a = oracle.prefill(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, f"C client m={m} k={k} n={n} bits={bits}")
