"""trellis_prefill_noalloc: the same layer with the workspace in a fixed
device array instead of memory the library allocates.

Its output must equal trellis_prefill's bit for bit (same kernels, same
partition, fixed summation order) and meet the oracle's tolerance, on two
calls in a row, the second with a smaller input; a call whose workspace does
not fit the fixed scratch is rejected before any GPU work.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from tests.helpers import assert_prefill_close, from_dev_bf16, to_dev_bf16, to_dev_codes
from workloads import generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def both(x, codes, scales, bits):
    import torch

    xd, cd, sd = to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales)
    m, n = x.shape[0], codes.shape[0]
    out_na = torch.full((m, n), -1.0, dtype=torch.bfloat16, device=xd.device)
    tp.prefill_noalloc(xd, cd, sd, bits, out_na)
    ref = tp.prefill(xd, cd, sd, bits)
    torch.cuda.synchronize()
    return from_dev_bf16(out_na), from_dev_bf16(ref)


def test_noalloc_matches_prefill_two_calls_shrinking():
    cases = [(8, 5120, 17408, 4, 9901), (5, 1024, 2004, 3, 9902)]
    for m, k, n, bits, seed in cases:
        print(f"noalloc m={m} k={k} n={n} bits={bits}", flush=True)
        x, codes, scales = generate(m, k, n, bits, seed=seed)
        got, ref = both(x, codes, scales, bits)
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} outputs differ from trellis_prefill"
        y, a = oracle.prefill_parallel(x, codes, scales, k, bits)
        assert_prefill_close(got, y, a, f"noalloc m={m} k={k} n={n}")


def test_noalloc_down_projection_shape():
    # K panels: every tile goes through the scratch's partial slots.
    m, k, n, bits = 15, 17408, 5120, 4
    print("noalloc down projection", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=9903, x_kind="silu_mul")
    got, ref = both(x, codes, scales, bits)
    assert np.array_equal(got, ref)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    import torch

    x = torch.zeros((5, 5120), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((5, 16), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((16, 640), dtype=torch.int32, device="cuda")
    scales = torch.zeros((16,), dtype=torch.bfloat16, device="cuda")
    # N = 2^22 at K = 5120 would need far more than 31 MiB of partial tiles;
    # the call is refused before anything is launched, so the (too small)
    # buffers are never read.
    g = tp.geom(1 << 22, 5120, 4)
    rc = tp.load_library().trellis_prefill_noalloc(x.data_ptr(), 5, codes.data_ptr(), scales.data_ptr(), g,
                                                   out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == tp.E_SCRATCH
    assert "scratch" in tp.status_string(rc)
